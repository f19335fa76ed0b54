// Pipelined bf16 grouped GEMM for gfx950 (expert up / down passes).
//
// Same contract as the first bf16 path in grouped_gemm.hip (C = epi(A B^T)
// over ragged groups, see GemmArgs), built for throughput:
//  * operands go global -> LDS directly (global_load_lds_dwordx4: each lane's
//    16 bytes land at M0 + 16 * lane), no register staging;
//  * an NS-stage LDS ring of K = 32 SUB slabs (SUB = 1 or 2), loads issued NS-1
//    stages ahead, one barrier per stage;
//  * stage rows are 64 SUB bytes with their 16-byte chunks permuted per row
//    (swz) so MFMA operand reads run conflict-free, while each 4 SUB lanes of a
//    load still fetch one row's 64 SUB contiguous bytes (SUB = 2: whole
//    128-byte cache lines);
//  * block tile BM x BN, WGM x WGN waves, each wave (BM/WGM) x (BN/WGN) of
//    MF x MF MFMA tiles: v_mfma_f32_32x32x16_bf16 (MF = 32) wherever the wave
//    tile is a multiple of 32, else v_mfma_f32_16x16x32_bf16 (MF = 16).  On
//    gfx950 both issue at the dense bf16 rate (16 and 32 cycles: 2.29 and
//    2.47 PFLOP/s in asm register-operand loops on MI355X), for the same
//    operand bytes per flop at a given wave tile;
//  * the output is staged through LDS in MF WGM-row chunks for 16-byte stores.
// Requires K % (32 SUB) == 0 (and, for S > 1, Kseg % (32 SUB) == 0).

#include <type_traits>

#include "common.h"
#include "internal.h"
#include "gemm_tiles.h"
#include "lds_ring.h"

namespace moe {

template <int BM, int BN, int WGM, int WGN, int NS, int SUB, bool SEG, int MF>
struct V2 {
  static constexpr int NW = WGM * WGN, NT = 64 * NW;     // waves, threads
  static constexpr int WM = BM / WGM, WN = BN / WGN;     // wave tile
  static constexpr int TM = WM / MF, TN = WN / MF;       // MFMA tiles per wave
  static constexpr int KQ = MF == 16 ? 1 : 2;            // MFMA k-steps per 32 of K
  static constexpr int RB = 64 * SUB;                    // bytes per stage row
  static constexpr int KS = 32 * SUB;                    // K per stage
  static constexpr int RPI = 1024 / RB;                  // rows per load instruction
  // load instructions per wave per stage: every wave issues the same number
  // (the vmcnt waits count them).  When BM + BN rows do not split evenly the
  // surplus instructions (whole RPI-row groups past row BM + BN) load into one
  // shared 1 KB dummy slot that is never read, so the stages stay unpadded.
  static constexpr int LPW = (BM + BN + RPI * NW - 1) / (RPI * NW);
  static constexpr bool PAD = LPW * NW * RPI > BM + BN;
  static constexpr int SLAB = (BM + BN) * RB;            // bytes per stage
  static constexpr int SR = MF * WGM;                    // output rows staged per pass
  // staged row (bf16): padded where the SR rows then still fit one stage
  // buffer (16 x 16 tiles), always for 32 x 32 tiles; SPLIT: the SR rows do
  // not fit one buffer, and wave row wm's MF rows sit in stage buffer wm
  static constexpr int LDC = (MF == 32 || SR * (BN + 8) * 2 <= SLAB) ? BN + 8 : BN;
  static constexpr bool SPLIT = SR * LDC * 2 > SLAB;
  static constexpr int SQ_BUF = SPLIT ? WGM : 1;         // stage buffer of the row sums of squares
  static_assert(MF == 16 || MF == 32, "16 x 16 x 32 or 32 x 32 x 16 MFMA");
  static_assert(SUB == 1 || SUB == 2, "32- or 64-wide K stages");
  static_assert(BM % (MF * WGM) == 0 && BN % (MF * WGN) == 0, "wave tiles are whole MFMA tiles");
  static_assert(!SPLIT || (MF * LDC * 2 <= SLAB && NS > WGM), "staged output rows must fit the stage buffers");
  static_assert(WGN * BM * 4 <= SLAB, "the row sums of squares fit one stage buffer");
  static_assert((BM + BN) % RPI == 0, "a load instruction covers whole rows of one kind");
  static_assert(NS >= 2 && NS <= 6, "2 to 6 stages");
};

// One LDS array per stage: distinct objects let the compiler see that reading
// one stage does not alias the loads in flight into the others.
// ACT: the epilogue activation, fixed at compile time (-1: none; p.act must match).
// MINB blocks must fit on a CU at once.  A block's waves are dealt over the
// four SIMDs from the first, so each block can put ceil(NW / 4) waves on one
// SIMD: the register budget is set for MINB times that many waves per SIMD
// (six-wave blocks otherwise get a budget for three and run one block per CU).
template <int MF>
using AccT = typename std::conditional<MF == 16, f32x4_t, f32x16_t>::type;

// One MFMA: weight operand first, so each lane holds consecutive columns of
// one output row (MF = 16: row lane % 16, columns 4 (lane / 16) + r; MF = 32:
// row lane % 32, columns 8 (r / 4) + 4 (lane / 32) + r % 4).
template <int MF>
__device__ __forceinline__ void mfma_step(const bf16x8_t& w, const bf16x8_t& a, AccT<MF>& c) {
  if constexpr (MF == 16) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w, a, c, 0, 0, 0);
  else c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w, a, c, 0, 0, 0);
}

template <int BM, int BN, int WGM, int WGN, int NS, int SUB, int MINB, bool SEG, int ACT, int MF>
__global__ __launch_bounds__(64 * WGM * WGN)
__attribute__((amdgpu_waves_per_eu(MINB * ((WGM * WGN + 3) / 4))))
void gemm_bf16_v2_kernel(GemmArgs p) {
  using C = V2<BM, BN, WGM, WGN, NS, SUB, SEG, MF>;
  constexpr int TM = C::TM, TN = C::TN, LPW = C::LPW, NW = C::NW, NT = C::NT, KQ = C::KQ;
  using Acc = AccT<MF>;
  // ping-pong schedule (two groups of four waves, one of each a SIMD)
  constexpr bool PP = BM == 256 && BN == 256 && WGM == 2 && WGN == 4 && NS == 4 && SUB == 1;
  __shared__ __attribute__((aligned(1024))) char st0[C::SLAB];
  __shared__ __attribute__((aligned(1024))) char st1[C::SLAB];
  __shared__ __attribute__((aligned(1024))) char st2[NS > 2 ? C::SLAB : 16];
  __shared__ __attribute__((aligned(1024))) char st3[NS > 3 ? C::SLAB : 16];
  __shared__ __attribute__((aligned(1024))) char st4[NS > 4 ? C::SLAB : 16];
  __shared__ __attribute__((aligned(1024))) char st5[NS > 5 ? C::SLAB : 16];
  __shared__ __attribute__((aligned(1024))) char st_pad[C::PAD ? 1024 : 16];
  __shared__ int s_info[4];
  char* const stages[6] = {st0, st1, st2, st3, st4, st5};

  const int n_tiles = (p.N + BN - 1) / BN;
  const Tile tl = find_tile<BM>(p.group_offset, p.G, p.dense_M, p.max_rows, n_tiles, s_info, p.n_major);
  if (tl.M <= 0) return;  // uniform

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: M0 for the loads is scalar arithmetic
  const int wm = wave / WGN, wn = wave % WGN;
  const int N = p.N, K = p.K;
  const int n0 = tl.nt * BN;
  const bf16_t* A = (const bf16_t*)p.A;
  const bf16_t* B = (const bf16_t*)p.B;

  // ---- this lane's load slots: instruction j = wave + NW i fills stage rows
  // RPI j .. RPI j + RPI - 1 (1 KB); lane l fills row RPI j + l / (4 SUB),
  // physical chunk l % (4 SUB), so each 4 SUB lanes fetch one row's 64 SUB
  // contiguous bytes.  Rows past BM + BN (the surplus instructions) read a
  // clamped weight row into the dummy slot.
  // Gathered rows: every slot's row index is loaded before any address is
  // formed (weight slots load the tile's first index, unused), so the loads
  // share one wait; loaded under the per-slot branch each got its own.
  int64_t arow[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int row = C::RPI * (wave + NW * i) + lane / (4 * SUB);
    arow[i] = tl.row0 + (row < BM ? (row < tl.M ? row : tl.M - 1) : 0);
  }
  if (p.a_rows != nullptr) {  // uniform
    int ai[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) ai[i] = p.a_rows[arow[i]];
#pragma unroll
    for (int i = 0; i < LPW; ++i) arow[i] = ai[i];
  }
  const bf16_t* src[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int row = C::RPI * (wave + NW * i) + lane / (4 * SUB);
    const int chunk = (lane % (4 * SUB)) ^ swz_mf<SUB, MF>(row);  // logical chunk stored here
    if (row < BM) {
      src[i] = A + arow[i] * K + chunk * 8;
    } else {
      const int nr = row - BM;
      const int n = (n0 + nr < N) ? n0 + nr : N - 1;
      src[i] = SEG ? B + (int64_t)n * p.Kseg + chunk * 8
                   : B + ((int64_t)tl.g * N + n) * K + chunk * 8;
    }
  }
  const int nk = K / C::KS;
  auto issue = [&](int kt, int stage) {
    const int k = (kt < nk ? kt : nk - 1) * C::KS;  // past the end: harmless reload
    char* base = stages[stage];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int row0 = C::RPI * (wave + NW * i);
      int64_t off = k;
      if (SEG && row0 >= BM) {
        const int s = k / p.Kseg;
        off = (int64_t)s * N * p.Kseg + (k - s * p.Kseg);
      }
      char* dst = (C::PAD && row0 >= BM + BN) ? st_pad : base + row0 * C::RB;  // uniform
      __builtin_amdgcn_global_load_lds((const void*)(src[i] + off), (lds_ptr_t)dst, 16, 0, 0);
    }
  };

  Acc acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 4 * (MF / 16) * (MF / 16); ++r) acc[i][j][r] = 0.f;

  // operand read offsets (bytes within a stage): lane (fr, fc) reads row fr
  // of its MF-row tile at logical k-chunk 4 h + fc (MF = 16) or 4 h + 2 q + fc
  // (MF = 32, k-step q) of sub-slab h
  const int fr = lane % MF, fc = lane / MF;

  // this lane's bias columns (unsegmented bias), all loaded together (columns
  // past N read column N - 4, unused): before the K loop when the register
  // budget allows (at most four waves a SIMD, counting a wave holding more
  // than four groups as more), so the epilogue does not wait on them, else at
  // the start of the epilogue
  // (MF = 16: one group of four columns per N tile; MF = 32: four groups)
  constexpr int CG = MF == 16 ? 1 : 4;  // column groups of four a lane holds per N tile
  constexpr bool BIAS_EARLY = MINB * ((NW + 3) / 4) * (MF == 16 ? 1 : (TN * CG + 3) / 4) <= 4;
  const bf16_t* bias = (const bf16_t*)p.bias;
  uint2 bpre[TN][CG];
  auto col_of = [&](int j, int g) { return n0 + wn * C::WN + j * MF + (MF == 16 ? fc * 4 : 8 * g + 4 * fc); };
  auto load_bias = [&]() {
    if (!SEG && bias != nullptr) {  // uniform
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int g = 0; g < CG; ++g) {
          const int n = col_of(j, g);
          bpre[j][g] = *(const uint2*)(bias + (int64_t)tl.g * N + (n < N ? n : N - 4));
        }
    }
  };
  if constexpr (BIAS_EARLY) load_bias();
  // Row tile i's offsets differ from tile 0's by the constant i MF RB: the
  // permutation of rows R and R + MF i is the same for every placement used
  // (the bits it takes from R lie below MF), so one base per (h, q) is kept
  // and the tile offset folds into the read's immediate.
  int a_rd0[SUB][KQ], b_rd0[SUB][KQ];
#pragma unroll
  for (int h = 0; h < SUB; ++h) {
#pragma unroll
    for (int q = 0; q < KQ; ++q) {
      const int ch = 4 * h + (MF == 16 ? fc : 2 * q + fc);
      const int Ra = wm * C::WM + fr, Rb = BM + wn * C::WN + fr;
      a_rd0[h][q] = Ra * C::RB + ((ch ^ swz_mf<SUB, MF>(Ra)) << 4);
      b_rd0[h][q] = Rb * C::RB + ((ch ^ swz_mf<SUB, MF>(Rb)) << 4);
    }
  }
  auto a_at = [&](const char* base, int h, int q, int i) {
    return *(const bf16x8_t*)(base + a_rd0[h][q] + i * MF * C::RB);
  };
  auto b_at = [&](const char* base, int h, int q, int j) {
    return *(const bf16x8_t*)(base + b_rd0[h][q] + j * MF * C::RB);
  };
  if constexpr (PP) {
    // Ping-pong: waves 0-3 (group 0) and 4-7 (group 1) put one wave of each
    // group on every SIMD.  Every wave runs the same loop, per stage j:
    //   MEM(j): refill stage j - 1's buffer with this wave's share of stage
    //           j + NS - 1, read stage j's operands, wait for its share of
    //           stage j + 1; barrier
    //   MUL(j): multiply stage j; barrier
    // and group 1 passes one extra barrier before the loop (group 0 one
    // after it), so barrier arrivals pair group 0's MUL with group 1's MEM
    // and the other way round: one wave a SIMD multiplies while the other
    // loads and reads.  Stage j is read by group 0 between barriers 2j and
    // 2j + 1 and by group 1 between 2j + 1 and 2j + 2, so its buffer is free
    // from barrier 2j + 2, where both groups' MEM(j + 1) start; every share of
    // stage j + 1 is waited for before barrier 2j + 1 (group 0) or 2j + 2
    // (group 1), ahead of both groups' reads of it.
    const int grp = wave >> 2;
    bf16x8_t fa[KQ][TM], fb[KQ][TN];
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) issue(s, s);
    wait_vmcnt<(NS - 2) * LPW>();  // stage 0
    slab_barrier();
    if (grp == 1) slab_barrier();
    auto pp_step = [&](int kt, int stage) {
      __builtin_amdgcn_sched_barrier(0);
      issue(kt + NS - 1, (stage + NS - 1) % NS);
      const char* base = stages[stage];
#pragma unroll
      for (int q = 0; q < KQ; ++q) {
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[q][i] = a_at(base, 0, q, i);
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[q][j] = b_at(base, 0, q, j);
      }
      wait_vmcnt<(NS - 2) * LPW>();  // this wave's share of stage kt + 1
      slab_barrier();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < KQ; ++q)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) mfma_step<MF>(fb[q][j], fa[q][i], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
      slab_barrier();
    };
    int kt = 0;
    for (; kt + NS <= nk; kt += NS) {
#pragma unroll
      for (int s = 0; s < NS; ++s) pp_step(kt + s, s);
    }
#pragma unroll
    for (int s = 0; s < NS; ++s)
      if (kt + s < nk) pp_step(kt + s, s);
    if (grp == 0) slab_barrier();
  } else {
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) issue(s, s);

  auto step = [&](int kt, int stage) {
    wait_vmcnt<(NS - 2) * LPW>();   // this wave's loads of stage kt have landed
    slab_barrier();                  // ... and every other wave's
    issue(kt + NS - 1, (stage + NS - 1) % NS);
    const char* base = stages[stage];
#pragma unroll
    for (int h = 0; h < SUB; ++h)
#pragma unroll
      for (int q = 0; q < KQ; ++q) {
        bf16x8_t a[TM], b[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) a[i] = a_at(base, h, q, i);
#pragma unroll
        for (int j = 0; j < TN; ++j) b[j] = b_at(base, h, q, j);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) mfma_step<MF>(b[j], a[i], acc[i][j]);
      }
  };

  int kt = 0;
  for (; kt + NS <= nk; kt += NS) {
#pragma unroll
    for (int s = 0; s < NS; ++s) step(kt + s, s);
  }
#pragma unroll
  for (int s = 0; s < NS; ++s)
    if (kt + s < nk) step(kt + s, s);
  }
  wait_vmcnt<0>();
  __syncthreads();

  // ---- epilogue: lane holds, for each row tile i and N tile j, row
  // m = wm WM + i MF + fr and CG groups of four consecutive columns
  // n = col_of(j, g) + r (the weight operand goes first; N % 8 == 0 puts all
  // four of a group in range or none)
  if constexpr (!BIAS_EARLY) load_bias();
  float bcol[TN][CG][4];
  bool ncol_ok[TN][CG];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int g = 0; g < CG; ++g) {
      const int n = col_of(j, g);
      ncol_ok[j][g] = n < N;
#pragma unroll
      for (int r = 0; r < 4; ++r) bcol[j][g][r] = 0.f;
      if (ncol_ok[j][g] && bias != nullptr) {
        if (SEG) {
          for (int q = 0; q < p.S; ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r) bcol[j][g][r] += bf16_to_f32(bias[(int64_t)q * N + n + r]);
        } else {
          const uint2 bb = bpre[j][g];
          bcol[j][g][0] = __uint_as_float(bb.x << 16);
          bcol[j][g][1] = __uint_as_float(bb.x & 0xffff0000u);
          bcol[j][g][2] = __uint_as_float(bb.y << 16);
          bcol[j][g][3] = __uint_as_float(bb.y & 0xffff0000u);
        }
      }
    }
  const bool want_sq = p.sq_part != nullptr;
  if (p.out_f32) {
    // fp32 result straight from the accumulators: 16 contiguous bytes a lane
    float* Cf = (float*)p.C;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int g = 0; g < CG; ++g) {
          const int m = wm * C::WM + i * MF + fr;
          const int n = col_of(j, g);
          f32x4_t v;
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = act_static<ACT>(acc[i][j][4 * g + r] + bcol[j][g][r]);
          if (m < tl.M && ncol_ok[j][g]) *(f32x4_t*)(Cf + (tl.row0 + m) * (int64_t)N + n) = v;
        }
    return;
  }
  bf16_t* Cg = (bf16_t*)p.C;
  float (*s_sq)[BM] = (float (*)[BM])stages[C::SQ_BUF];  // [WGN][BM]; the ring is idle now
  // Pass i stages row tile i of every wave row and stores it: staging row
  // MF wm + q holds tile row wm WM + MF i + q, in stage buffer 0 or, split, in
  // stage buffer wm (row q there).
  bf16_t* Cs = C::SPLIT ? (bf16_t*)stages[wm] : (bf16_t*)st0 + wm * MF * C::LDC;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int g = 0; g < CG; ++g) {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[r] = act_static<ACT>(acc[i][j][4 * g + r] + bcol[j][g][r]);
          if (want_sq && ncol_ok[j][g]) rs += v[r] * v[r];
        }
        uint2 pk;
        pk.x = pack_bf16x2(v[0], v[1]);
        pk.y = pack_bf16x2(v[2], v[3]);
        *(uint2*)(Cs + fr * C::LDC + (col_of(j, g) - n0)) = pk;
      }
    if (want_sq) {
      // the row's lanes (four for MF = 16, two for MF = 32), then (below) the
      // WGN wave columns in order
      if constexpr (MF == 16) rs += __int_as_float(xor_lane<16>(__float_as_int(rs)));
      rs += __int_as_float(xor_lane<32>(__float_as_int(rs)));
      if (fc == 0) s_sq[wn][wm * C::WM + i * MF + fr] = rs;
    }
    __syncthreads();
    constexpr int VPR = BN / 8;  // 16-byte vectors per staged row
#pragma unroll
    for (int v = tid; v < C::SR * VPR; v += NT) {
      const int sr = v / VPR, cv = v % VPR;
      const int m = (sr / MF) * C::WM + i * MF + (sr % MF);
      const int n = n0 + cv * 8;
      const bf16_t* row = C::SPLIT ? (const bf16_t*)stages[sr / MF] + (sr % MF) * C::LDC
                                   : (const bf16_t*)st0 + sr * C::LDC;
      if (m < tl.M && n < N) store16_agent(Cg + (tl.row0 + m) * (int64_t)N + n, *(const vec16*)(row + cv * 8));
    }
    __syncthreads();
  }
  if (want_sq)
    for (int m = tid; m < tl.M; m += NT) {
      float sum = 0.f;
      for (int q = 0; q < WGN; ++q) sum += s_sq[q][m];
      p.sq_part[(tl.row0 + m) * (int64_t)n_tiles + tl.nt] = sum;
    }
}

template <int BM, int BN, int WGM, int WGN, int NS, int SUB, int MINB, int MF>
static hipError_t launch_v2(const GemmArgs& a, hipStream_t st) {
  const int64_t rows = a.group_offset ? a.max_rows : a.dense_M;
  if (rows <= 0) return hipSuccess;
  const int64_t mt = (rows + BM - 1) / BM + (a.group_offset ? a.G : 0);
  const dim3 grid((unsigned)grid_blocks(mt, (a.N + BN - 1) / BN));
  const dim3 block(64 * WGM * WGN);
#define MOE_V2_LAUNCH(SEGV, ACTV) \
  hipLaunchKernelGGL((gemm_bf16_v2_kernel<BM, BN, WGM, WGN, NS, SUB, MINB, SEGV, ACTV, MF>), grid, block, 0, st, a)
#define MOE_V2_BY_ACT(SEGV)                                  \
  switch (a.act) {                                           \
    case ACT_RELU: MOE_V2_LAUNCH(SEGV, ACT_RELU); break;     \
    case ACT_GELU: MOE_V2_LAUNCH(SEGV, ACT_GELU); break;     \
    case ACT_SWISH: MOE_V2_LAUNCH(SEGV, ACT_SWISH); break;   \
    default: MOE_V2_LAUNCH(SEGV, -1); break;                 \
  }
  if (a.S > 1) {
    MOE_V2_BY_ACT(true);
  } else {
    MOE_V2_BY_ACT(false);
  }
#undef MOE_V2_BY_ACT
#undef MOE_V2_LAUNCH
  return hipGetLastError();
}

bool gemm_v2_supported(const GemmArgs& a) {
  return a.K % 32 == 0 && (a.S <= 1 || a.Kseg % 32 == 0);
}

bool gemm_v2_wide_k(const GemmArgs& a) { return a.K % 64 == 0 && (a.S <= 1 || a.Kseg % 64 == 0); }

// Eight waves (2 x 4) per block and a 3-stage ring: with two or three blocks
// resident per CU each SIMD holds four or more waves, which hides the LDS and
// barrier latency of one slab behind another wave's MFMAs (measured on
// MI355X: 10-35 % faster than four waves with a 4-stage ring on the expert
// shapes, bit-identical results).  The 144-row tiles use twelve waves in
// 3 x 4 (48 x 32 each) with 64-wide K stages: a 2-stage ring when two blocks
// share a CU, a 4-stage ring when one block runs alone (measured on MI355X on
// the 8-expert default passes: up 23.9 -> 20.2 us, down 17.8 -> 16.2 us
// against six waves in 3 x 2; the extra waves hide the LDS and load latency
// that one or two six-wave blocks leave exposed).  Without 64-wide K they use
// six waves in 3 x 2 and 32-wide stages.  Over several waves of 256 x 256
// tiles a 4-stage ring of 32-wide stages (128 KB) keeps three stages of loads
// in flight where the 2-stage 64-wide ring keeps one (measured on MI355X: 128
// experts of 2048 rows at d 4096, F 1536: up 3646 -> 3284 us, down 3677 ->
// 3449 us; 64 experts of 768 rows at d 2048, F 1408: down 380 -> 350 us).
// Every configuration accumulates K in the same order, so all give the same
// bits.
hipError_t launch_gemm_bf16_v2(const GemmArgs& a, int tile, hipStream_t st) {
  // Every tile runs the 16 x 16 x 32 MFMA: on the expert shapes the 32 x 32 x
  // 16 form measured slower in these loops (MI355X, 128 experts of 2048 rows
  // at d 4096, F 1536, up pass: 256 x 256 tiles 933 against 1073 TFLOP/s,
  // 64-wide 2-stage ring 1009, no ping-pong 986, ping-pong on half stages of
  // a 2-stage 64-wide ring 667).  Neither is bound by the matrix pipe: the
  // waves stall on operand reads, stage loads and the per-tile epilogue.
  // 256 x 256 tiles go to the persistent kernel (gemm_bf16_persist.hip)
  // where it supports the pass; this one keeps the rest.  (With its half-
  // height and half-width tile modes the persistent kernel also took the
  // fine-grained up pass, N = 1408, from 385 to 357 us before the half-width
  // mode.)
  if (tile == 513)
    return gemm_persist_supported(a) ? launch_gemm_bf16_persist(a, st)
                                     : launch_v2<256, 256, 2, 4, 4, 1, 1, 16>(a, st);
  if (tile == 256) return launch_v2<256, 128, 2, 4, 3, 1, 2, 16>(a, st);
  if (tile == 144)
    return gemm_v2_wide_k(a) ? launch_v2<144, 128, 3, 4, 2, 2, 2, 16>(a, st)
                             : launch_v2<144, 128, 3, 2, 3, 1, 2, 16>(a, st);
  if (tile == 145) return launch_v2<144, 128, 3, 4, 4, 2, 1, 16>(a, st);
  // 128 x 256 tiles with K % 64 == 0 take 64-wide stages (whole 128-byte
  // lines a row) in a 3-stage ring, one block a CU: the switch layer's up
  // pass (weight rows of 2 KB streamed in K slabs) 158-160 -> 154 us against
  // two blocks a CU on 32-wide stages
  if (tile == 257)
    return gemm_v2_wide_k(a) ? launch_v2<128, 256, 2, 4, 3, 2, 1, 16>(a, st)
                             : launch_v2<128, 256, 2, 4, 3, 1, 2, 16>(a, st);
  if (tile == 259) return launch_v2<128, 128, 2, 4, 4, 2, 1, 16>(a, st);
  if (tile == 64) return launch_v2<128, 64, 2, 2, 4, 1, 2, 16>(a, st);
  return launch_v2<128, 128, 2, 4, 3, 1, 2, 16>(a, st);
}

}  // namespace moe
