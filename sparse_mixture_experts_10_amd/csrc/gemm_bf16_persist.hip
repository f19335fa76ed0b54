// Persistent bf16 grouped GEMM for the large expert passes (256 x 256 tiles).
//
// Same contract as the other bf16 paths (C = epi(A B^T) over ragged groups,
// see GemmArgs), for passes with several waves of 256 x 256 tiles, K a
// multiple of 32 SUB, one K segment, bf16 output:
//  * one block of four waves per CU, each block walking its share of the
//    tile list (the list is dealt to the 8 XCDs in contiguous bands, as in
//    find_tile, and inside a band to the XCD's blocks round-robin);
//  * each wave owns a 128 x 128 output tile (8 x 8 v_mfma_f32_16x16x32_bf16
//    tiles, 256 accumulator registers in AGPRs) and software-pipelines its
//    K loop: while it multiplies one 32-wide step from one fragment set it
//    reads the next step into the other and issues the global -> LDS loads
//    (global_load_lds_dwordx4) of the stage NS ahead into the buffer the
//    previous stage left, one barrier per stage;
//  * a tile of at most 128 rows runs half-height (the four waves side by
//    side along N, 128 x 64 each) and one of at most 128 valid columns
//    half-width (stacked along M, 64 x 128 each): half the MFMAs, the same
//    loads;
//  * between tiles, the next tile's first NS stages are issued before the
//    finished tile's epilogue runs, so their latency hides behind it;
//  * the epilogue is per wave: bias (staged in LDS during the tile's K
//    loop), activation, optional row sums of squares, bf16 rows written
//    straight from registers as 16-byte stores (lanes exchange pieces by
//    permlane moves), with no block barrier until the row sums are
//    combined.  Outputs larger than the 256 MB Infinity Cache are stored
//    as eight whole 128-byte row lines a store (a further DPP exchange)
//    with the non-temporal hint: the pass never reads its output again,
//    and an output of gigabytes otherwise evicts the operand lines other
//    blocks still read from the XCD's L2 and competes for HBM.  Measured
//    on MI355X (large down pass, 2.1 GB out): without any output stores
//    the pass ran 20 % faster, with every store of an XCD aimed at one
//    128 KB region (no write-back, no eviction) 19 %, at an 8 MB region
//    (eviction, no HBM writes) 10 %; whole-line non-temporal stores gained
//    1-3 % over plain 64-byte row pieces (agent- or system-scope stores, and
//    non-temporal 64-byte pieces, were slower).  Smaller outputs, read back
//    from that cache by the next pass, keep plain 64-byte row pieces.
// The accumulation order over K is the same as every other configuration's
// (32-wide steps in order, each one MFMA), so C is bit-identical to theirs.
// Measured on MI355X (128 groups of 2048 rows, d 4096, F 1536): a non-
// persistent kernel of this shape spent 20-25 % of each block in the
// epilogue and 3-8 % waiting for its first stage, with every CU writing its
// tile back at the same moment.

#include <type_traits>

#include "common.h"
#include "internal.h"
#include "gemm_tiles.h"
#include "lds_ring.h"

namespace moe {

template <int SUB>
struct PCfg {
  static constexpr int BM = 256, BN = 256, NW = 4, NT = 256, WM = 128, WN = 128, MF = 16;
  static constexpr int TM = WM / MF, TN = WN / MF;           // 8 x 8 MFMA tiles a wave
  static constexpr int NS = SUB == 1 ? 4 : 2;               // stages in the LDS ring
  static constexpr int RB = 64 * SUB, KS = 32 * SUB;        // bytes per stage row, K per stage
  static constexpr int RPI = 1024 / RB;                     // rows per load instruction
  static constexpr int LPW = (BM + BN) / (RPI * NW);        // load instructions per wave per stage
  static constexpr int SLAB = (BM + BN) * RB;               // bytes per stage
  static constexpr int NMF = TM * TN;                       // MFMAs per 32-wide step
  static constexpr int NRD = TM + TN;                       // operand reads per 32-wide step
  static constexpr int kMaxG = 256;
  static_assert((BM + BN) % (RPI * NW) == 0, "load instructions cover whole stages");
  static_assert(NS * SLAB == 131072, "the ring takes 128 KB");
};

// One v_mfma_f32_16x16x32_bf16 with the accumulator tied to an AGPR quad.
// Written as asm so the 256 accumulator registers stay in one register file
// (as builtins the compiler moved them between AGPRs and VGPRs around every
// MFMA) and keep their written order (asm volatile).  The compiler does not
// know these are MFMAs: the wait states an MFMA result needs before another
// instruction reads it are added by hand where the accumulators are read.
__device__ __forceinline__ void mfma16_acc(const bf16x8_t& w, const bf16x8_t& a, f32x4_t& c) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(w), "v"(a));
}

// One accumulator element to a VGPR, read where it is used: as plain code
// the compiler copied all 256 accumulators to VGPRs at the end of the K loop
// and spilled the values the next tile needs (spill reloads wait for every
// memory operation in flight, the next tile's loads included).
__device__ __forceinline__ float acc_read(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

// NTS: outputs stored as whole 128-byte lines with the non-temporal hint
// (large outputs), else as plain 64-byte row pieces.
template <int SUB, int ACT, bool NTS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
void gemm_bf16_persist_kernel(GemmArgs p) {
  using C = PCfg<SUB>;
  constexpr int NS = C::NS, LPW = C::LPW, TM = C::TM, TN = C::TN, NMF = C::NMF, NRD = C::NRD;
  constexpr int BM = C::BM, BN = C::BN, NW = C::NW, MF = C::MF;
  // one LDS array per stage: distinct objects let the compiler see that
  // reading one stage does not alias the loads in flight into the others
  __shared__ __attribute__((aligned(1024))) char st0[C::SLAB];
  __shared__ __attribute__((aligned(1024))) char st1[C::SLAB];
  __shared__ __attribute__((aligned(1024))) char st2[NS > 2 ? C::SLAB : 16];
  __shared__ __attribute__((aligned(1024))) char st3[NS > 3 ? C::SLAB : 16];
  __shared__ __attribute__((aligned(16))) bf16_t s_bias[BN];           // bias of the tile's columns
  __shared__ float s_sq[NW][BM];                                     // row sums of squares per wave column
  __shared__ int s_pre[C::kMaxG + 1];                                // row-tile prefix over groups
  __shared__ int s_goff[C::kMaxG + 1];                               // group row offsets
  // ring slot s (s is a compile-time constant wherever this is called)
  auto slot = [&](int s) -> char* { return s == 0 ? st0 : s == 1 ? st1 : s == 2 ? st2 : st3; };

  // the wave index in a scalar register: the load slots' LDS addresses (M0)
  // are then scalar arithmetic, not a VGPR read back at every load
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int N = p.N, K = p.K;
  const int n_tiles = (N + BN - 1) / BN;
  const int nk = K / C::KS;
  const bf16_t* A = (const bf16_t*)p.A;
  const bf16_t* B = (const bf16_t*)p.B;
  const bf16_t* bias = (const bf16_t*)p.bias;
  const bool grouped = p.group_offset != nullptr;
  const int G = grouped ? p.G : 1;

  // ---- row-tile table (wave 0): s_pre[g] = row tiles of groups before g,
  // s_goff[g] = first row of group g
  if (wave == 0) {
    if (!grouped) {
      if (lane == 0) {
        s_pre[0] = 0;
        s_pre[1] = (int)((p.dense_M + BM - 1) / BM);
        s_goff[0] = 0;
        s_goff[1] = (int)p.dense_M;
      }
    } else {
      const int gpl = (G + 63) / 64;  // groups per lane (<= 4)
      const int g0 = lane * gpl;
      int lo[4], hi[4], local = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int g = g0 + q < G ? g0 + q : G - 1;
        lo[q] = p.group_offset[g];
        hi[q] = p.group_offset[g + 1];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (q < gpl && g0 + q < G) local += (hi[q] - lo[q] + BM - 1) / BM;
      int incl = local;
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        const int o = __shfl_up(incl, m, 64);
        if (lane >= m) incl += o;
      }
      int pre = incl - local;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int g = g0 + q;
        if (q < gpl && g < G) {
          s_pre[g] = pre;
          s_goff[g] = lo[q];
          pre += (hi[q] - lo[q] + BM - 1) / BM;
          if (g == G - 1) {
            s_pre[G] = pre;
            s_goff[G] = hi[q];
          }
        }
      }
    }
  }
  __syncthreads();
  // list positions fit 32 bits (checked by the launcher)
  const int total_m = __builtin_amdgcn_readfirstlane(s_pre[G]);
  const int total = total_m * n_tiles;
  const int band = (total + kXcds - 1) / kXcds;
  const int xcd = blockIdx.x % kXcds;
  const int first = blockIdx.x / kXcds, step = gridDim.x / kXcds;
  // The band's last round: when its tiles fill at most half of the XCD's
  // blocks and the K loop is long (K >= 4096), each is dealt as two
  // half-height pieces (rows 0 .. 127 and 128 .. 255, each in the
  // half-height mode), so the round takes about half a tile's time on twice
  // the blocks instead of a whole tile's on few.  (Measured on MI355X: large
  // up pass, K 4096, 3045 -> 3029 us; with K 1408-2048 the shorter last
  // round gained nothing, or lost up to 2 %.)
  // A piece computes its rows exactly as the whole tile would (same K
  // order); only its row sums of squares add four wave partials, not two.
  const int blen = total - xcd * band < band ? (total - xcd * band > 0 ? total - xcd * band : 0) : band;
  const int full_rounds = blen / step;
  const int rem = blen - full_rounds * step;
  const bool split_tail = 2 * rem <= step && K >= 4096;
  const int vlen = split_tail ? full_rounds * step + 2 * rem : blen;

  // tile of position i of this block's band, counting the last round's
  // pieces (M = 0: nothing to do there; M = -1: past the band's end); lane
  // values (each lane may ask for its own i)
  auto tile_core = [&](int i) {
    Tile tl;
    tl.g = 0; tl.row0 = 0; tl.M = -1; tl.nt = 0;
    if (i >= vlen) return tl;
    int piece = -1;  // 0, 1: the half of a split last-round tile
    int ib = i;
    if (split_tail && i >= full_rounds * step) {
      const int v = i - full_rounds * step;
      ib = full_rounds * step + v / 2;
      piece = v & 1;
    }
    const int L = xcd * band + ib;
    const int mt = L / n_tiles;
    int lo = 0, hi = G;  // s_pre[lo] <= mt < s_pre[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_pre[mid] <= mt) lo = mid;
      else hi = mid;
    }
    const int pre = s_pre[lo];
    const int tiles = s_pre[lo + 1] - pre;
    int r = mt - pre;
    tl.nt = L - mt * n_tiles;
    if (p.n_major) {
      const int l = L - pre * n_tiles;
      tl.nt = l / tiles;
      r = l - tl.nt * tiles;
    }
    const int Mg = s_goff[lo + 1] - s_goff[lo];
    tl.g = grouped ? lo : 0;
    tl.row0 = (int64_t)s_goff[lo] + (int64_t)r * BM;
    tl.M = Mg - r * BM < BM ? Mg - r * BM : BM;
    if (tl.row0 >= p.max_rows) tl.M = 0;
    else if (tl.row0 + tl.M > p.max_rows) tl.M = (int)(p.max_rows - tl.row0);
    if (piece >= 0) {
      if (tl.M <= BM / 2) {
        if (piece == 1) tl.M = 0;  // a half-height tile already: one piece
      } else {
        tl.row0 += (int64_t)piece * (BM / 2);
        tl.M = piece ? tl.M - BM / 2 : BM / 2;
      }
    }
    return tl;
  };
  // The block's tiles, positions first, first + step, ..., looked up once
  // into LDS by all threads together (one position a thread: a binary
  // search over the groups each); a tile transition then reads its entry
  // instead of searching (7 dependent LDS reads for 128 groups, about 1 % of
  // the large down pass).  Positions past the table's end are searched.
  constexpr int kTab = 256;
  __shared__ int4 s_tab[kTab];
  const int npos = vlen > first ? (vlen - first + step - 1) / step : 0;
  for (int q = tid; q < npos && q < kTab; q += C::NT) {
    const Tile t = tile_core(first + q * step);
    s_tab[q] = make_int4(t.g, (int)t.row0, t.M, t.nt);
  }
  __syncthreads();
  // the block's q-th tile; the same for every lane: kept in scalar registers
  auto tile_q = [&](int q) {
    Tile tl;
    if (q < kTab) {
      const int4 e = q < npos ? s_tab[q] : make_int4(0, 0, -1, 0);
      tl.g = e.x; tl.row0 = e.y; tl.M = e.z; tl.nt = e.w;
    } else {
      tl = tile_core(first + q * step);
    }
    tl.g = __builtin_amdgcn_readfirstlane(tl.g);
    tl.M = __builtin_amdgcn_readfirstlane(tl.M);
    tl.nt = __builtin_amdgcn_readfirstlane(tl.nt);
    tl.row0 = (int64_t)__builtin_amdgcn_readfirstlane((int)tl.row0);
    return tl;
  };

  // ---- per-tile load slots: instruction j = wave + NW i fills stage rows
  // RPI j .. RPI j + RPI - 1 (1 KB); lane l fills row RPI j + l / (4 SUB),
  // physical chunk l % (4 SUB) (its logical chunk permuted by swz), so each
  // 4 SUB lanes fetch one row's 64 SUB contiguous bytes
  // Slots i < NA hold A rows for every wave (RPI (wave + NW i) < BM), the
  // rest weight rows: decided by i alone, at compile time.
  constexpr int NA = LPW / 2;
  static_assert(C::RPI * NW * NA == BM && BM == BN, "the first half of the slots loads the A rows");
  const bf16_t* src[LPW];
  auto set_sources = [&](const Tile& tl) {
    int arow[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int row = C::RPI * (wave + NW * i) + lane / (4 * SUB);
      arow[i] = (int)tl.row0 + (row < tl.M ? row : tl.M - 1);
    }
    if (p.a_rows != nullptr) {
      int ai[NA];
#pragma unroll
      for (int i = 0; i < NA; ++i) ai[i] = p.a_rows[arow[i]];
#pragma unroll
      for (int i = 0; i < NA; ++i) arow[i] = ai[i];
    }
    const int n0 = tl.nt * BN;
    const bf16_t* const bt = B + (int64_t)tl.g * N * K;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int row = C::RPI * (wave + NW * i) + lane / (4 * SUB);
      const int chunk = (lane % (4 * SUB)) ^ swz_mf<SUB, MF>(row);
      if (i < NA) {
        src[i] = A + (int64_t)arow[i] * K + chunk * 8;
      } else {
        const int nr = row - BM;
        const int n = (n0 + nr < N) ? n0 + nr : N - 1;
        src[i] = bt + n * K + chunk * 8;
      }
    }
  };
  auto issue_one = [&](int kt, int stage, int i) {
    const int k = (kt < nk ? kt : nk - 1) * C::KS;  // past the end: harmless reload
    const int row0 = C::RPI * (wave + NW * i);
    __builtin_amdgcn_global_load_lds((const void*)(src[i] + k), (lds_ptr_t)(slot(stage) + row0 * C::RB), 16, 0, 0);
  };
  // the tile's first NS stages
  auto prologue = [&]() {
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int i = 0; i < LPW; ++i) issue_one(s, s, i);
  };
  // the tile's bias into LDS (waves 0 and 1, 64 lanes x two columns each;
  // N % 8 == 0 keeps both columns of a lane in range or neither, and columns
  // past N read N - 2, unused); read in the tile's epilogue
  auto load_bias = [&](const Tile& tl) {
    if (bias != nullptr && wave < 2) {
      const int n = tl.nt * BN + wave * 128 + 2 * lane;
      const bf16_t* bp = bias + (int64_t)tl.g * N + (n < N ? n : N - 2);
      __builtin_amdgcn_global_load_lds((const void*)bp, (lds_ptr_t)(&s_bias[wave * 128]), 4, 0, 0);
    }
  };

  // ---- operand reads: lane (fr, fc) reads row fr of its 16-row tile at
  // logical chunk 4 h + fc of sub-slab h; tile i's offset is i 16 RB.
  // Tile modes (M: the tile's rows, W: its columns inside N):
  //  * full: wave (wm, wn) takes rows 128 wm .. + 127, columns 128 wn .. + 127;
  //  * half-height (M <= 128): every wave takes rows 0 .. 127 against its
  //    own 64 columns, 64 wave .. + 63 (wave tile 128 x 64);
  //  * half-width (W <= 128, M > 128): every wave takes its own 64 rows,
  //    64 wave .. + 63, against columns 0 .. 127 (wave tile 64 x 128).
  // Either half mode has half the MFMAs of a full tile, whose other half
  // would multiply padding.  mode_rows / mode_cols: the wave's first row and
  // column.
  enum { M_FULL = 0, M_HALF_H = 1, M_HALF_W = 2 };
  // the half-width mode is built for 64-wide stages only (with the 32-wide
  // stages' deeper ring a third K loop spilled); the others run such tiles
  // in full mode
  constexpr bool kHalfW = SUB == 2;
  auto tile_mode = [&](int M, int nt) {
    return M <= BM / 2 ? M_HALF_H : (kHalfW && N - nt * BN <= BN / 2) ? M_HALF_W : M_FULL;
  };
  auto mode_row = [&](int mode) { return mode == M_FULL ? wm * C::WM : mode == M_HALF_H ? 0 : wave * (C::WM / 2); };
  auto mode_col = [&](int mode) { return mode == M_FULL ? wn * C::WN : mode == M_HALF_H ? wave * (C::WN / 2) : 0; };
  const int fr = lane % MF, fc = lane / MF;
  int a_rd0[SUB], b_rd0[SUB];
  auto set_reads = [&](int mode) {
    const int Ra = mode_row(mode) + fr;
    const int Rb = BM + mode_col(mode) + fr;
#pragma unroll
    for (int h = 0; h < SUB; ++h) {
      const int ch = 4 * h + fc;
      a_rd0[h] = Ra * C::RB + ((ch ^ swz_mf<SUB, MF>(Ra)) << 4);
      b_rd0[h] = Rb * C::RB + ((ch ^ swz_mf<SUB, MF>(Rb)) << 4);
    }
  };
  bf16x8_t fa[2][TM], fb[2][TN];
  // read r of a step: A fragments 0 .. tme - 1, then the B fragments
  auto read_one = [&](int set, const char* base, int h, int r, int tme) {
    if (r < tme) fa[set][r] = *(const bf16x8_t*)(base + a_rd0[h] + r * MF * C::RB);
    else fb[set][r - tme] = *(const bf16x8_t*)(base + b_rd0[h] + (r - tme) * MF * C::RB);
  };

  f32x4_t acc[TM][TN];

  // step h of stage kt (ring slot `stage`).  The waits count this tile's
  // stage loads only; the previous tile's output stores, issued after this
  // tile's first NS stages, then have to land too, which only waits longer.
  // mode_c: std::integral_constant<int, mode>.  Every mode issues the same
  // loads.
  auto sw_step = [&](auto mode_c, int kt, int stage, int h) {
    constexpr int MODE = decltype(mode_c)::value;
    constexpr int TMe = MODE == M_HALF_W ? TM / 2 : TM, TNe = MODE == M_HALF_H ? TN / 2 : TN;
    constexpr int NMFe = TMe * TNe, NRDe = TMe + TNe;
    const int cur = SUB == 1 ? stage & 1 : h;
    const bool last = h == SUB - 1;
    if (last) {
      wait_vmcnt<(NS - 2) * LPW>();  // this wave's share of stage kt + 1
      slab_barrier();
    }
    const char* nbase = last ? slot((stage + 1) % NS) : slot(stage);
    const int nh = last ? 0 : h + 1;
    // read r after MFMA 3 NMF r / (4 NRD), load l after MFMA 1 + 3 NMF l / (4 LPW):
    // all in the first three quarters of the step
#pragma unroll
    for (int t = 0; t < NMFe; ++t) {
      mfma16_acc(fb[cur][t % TNe], fa[cur][t / TNe], acc[t / TNe][t % TNe]);
#pragma unroll
      for (int r = 0; r < NRDe; ++r)
        if (3 * NMFe * r / (4 * NRDe) == t) read_one(cur ^ 1, nbase, nh, r, TMe);
      if (last) {
#pragma unroll
        for (int l = 0; l < LPW; ++l)
          if (1 + 3 * NMFe * l / (4 * LPW) == t) issue_one(kt + NS, stage, l);
      }
    }
  };
  // the tile's K loop from its stage 0 (landed and past the barrier).  The
  // accumulators are zeroed here and handed to the asm MFMAs through an
  // empty asm that takes them in AGPRs, so the writes come before the wait
  // states the first MFMA reading them needs; in half-height mode the unused
  // ones pass through an empty asm too, so both modes leave every
  // accumulator in an AGPR (otherwise the compiler kept the untouched ones
  // elsewhere and spilled).
  auto k_loop = [&](auto mode_c) {
    constexpr int MODE = decltype(mode_c)::value;
    constexpr int TMe = MODE == M_HALF_W ? TM / 2 : TM, TNe = MODE == M_HALF_H ? TN / 2 : TN;
    constexpr int NRDe = TMe + TNe;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        asm volatile("" : "+a"(acc[i][j]));
      }
    asm volatile("s_nop 7");
#pragma unroll
    for (int r = 0; r < NRDe; ++r) read_one(0, slot(0), 0, r, TMe);
    int kt = 0;
    for (; kt + NS <= nk; kt += NS) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int h = 0; h < SUB; ++h) sw_step(mode_c, kt + s, s, h);
    }
#pragma unroll
    for (int s = 0; s < NS; ++s)
      if (kt + s < nk) {
#pragma unroll
        for (int h = 0; h < SUB; ++h) sw_step(mode_c, kt + s, s, h);
      }
    if constexpr (MODE != M_FULL) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          if (i >= TMe || j >= TNe) asm volatile("" : "+a"(acc[i][j]));
    }
  };

  // ---- the tile loop
  int it = 0;  // the block's tile count so far
  Tile tl = tile_q(it);
  while (tl.M == 0) tl = tile_q(++it);
  if (tl.M < 0) return;  // uniform
  set_sources(tl);
  load_bias(tl);
  prologue();
  for (;;) {
    // stage 0 landed (at most the NS - 1 younger stages' loads in flight:
    // the previous tile's output stores, younger still, are partly drained)
    wait_vmcnt<(NS - 1) * LPW>();
    slab_barrier();
    // the tile's mode (uniform)
    const int mode = tile_mode(tl.M, tl.nt);
    set_reads(mode);
    if (mode == M_HALF_H) {
      k_loop(std::integral_constant<int, M_HALF_H>{});
    } else if (mode == M_HALF_W) {
      if constexpr (kHalfW) k_loop(std::integral_constant<int, M_HALF_W>{});
    } else {
      k_loop(std::integral_constant<int, M_FULL>{});
    }
    // MFMA results need up to 18 wait states before other instructions read them
    asm volatile("s_nop 7");
    asm volatile("s_nop 7");
    asm volatile("s_nop 7");

    // ---- every stage load of this tile has landed and been read (and the
    // harmless reloads past its end), and so has its bias: once every wave
    // is here the ring is free for the next tile's first loads
    const Tile cur_t = tl;
    do tl = tile_q(++it); while (tl.M == 0);
    wait_vmcnt<0>();
    __syncthreads();
    if (tl.M > 0) {
      set_sources(tl);
      prologue();
    }

    // ---- epilogue of cur_t: lane holds, for row tile i and column tile j,
    // row r0 + 16 i + fr and columns c0 + 16 j + 4 fc + r, with r0, c0 the
    // wave's first row and column in the tile's mode
    const int n0 = cur_t.nt * BN;
    const bool want_sq = p.sq_part != nullptr;
    auto epilogue = [&](auto mode_c) {
      constexpr int MODE = decltype(mode_c)::value;
      constexpr int TMe = MODE == M_HALF_W ? TM / 2 : TM, TNe = MODE == M_HALF_H ? TN / 2 : TN;
      const int r0 = mode_row(MODE), c0 = mode_col(MODE);
      // the wave column whose row sums this wave writes
      const int sq_col = MODE == M_FULL ? wn : MODE == M_HALF_H ? wave : 0;
      float bc[TNe][4];
      bool ok[TNe];
#pragma unroll
      for (int j = 0; j < TNe; ++j) {
        const int c = c0 + j * MF + 4 * fc;  // column within the tile
        ok[j] = n0 + c < N;
        if (bias != nullptr) {
          const uint2 bb = *(const uint2*)(&s_bias[c]);
          bc[j][0] = __uint_as_float(bb.x << 16);
          bc[j][1] = __uint_as_float(bb.x & 0xffff0000u);
          bc[j][2] = __uint_as_float(bb.y << 16);
          bc[j][3] = __uint_as_float(bb.y & 0xffff0000u);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) bc[j][r] = 0.f;
        }
      }
      // Register-direct stores.  Lanes fc and fc ^ 1 (lane and lane ^ 16)
      // pair up over two neighbouring column tiles 2 q, 2 q + 1: the even one
      // keeps its four columns of tile 2 q and takes its partner's four of
      // the same tile, the odd one takes its partner's four of tile 2 q + 1
      // and keeps its own, so each holds 8 consecutive columns (16 bytes) of
      // its row: lane fc covers columns 32 q + {0, 16, 8, 24}[fc] .. + 7, the
      // four lanes of a row 64 contiguous bytes.  Lanes fr and fr ^ 8 then
      // trade pieces so that each store writes eight whole 128-byte row
      // lines (below).  No LDS round trip.
      // Addresses: the tile's first element (uniform) plus a 32-bit byte
      // offset, the lane's part fixed and the step's part uniform (64-bit
      // per-store addresses were all formed up front and spilled, their
      // reloads waiting for the next tile's loads); the row check is the
      // lane's fixed row against a uniform bound.
      char* const cbase = (char*)((bf16_t*)p.C + cur_t.row0 * (int64_t)N + n0);
      // the lane's store columns (before + 64 p2) and row (before + 8 h)
      // the lane's store row and columns (whole lines: before + 8 h, + 64 p2;
      // row pieces: before + 32 q)
      const int colbase = ((fc & 1) ? 16 + 4 * (fc - 1) : 4 * fc) + (NTS ? 32 * (fr >> 3) : 0);
      const int lrow = NTS ? (fr & 7) : fr;
      const uint32_t lane_off = (uint32_t)(((r0 + lrow) * N + c0 + colbase) * 2);
      const int lane_row = r0 + lrow;
#pragma unroll
      for (int i = 0; i < TMe; ++i) {
        // one row tile at a time: kept from hoisting the next tile's
        // accumulator reads, which would need 256 registers at once (spills,
        // whose reloads wait for every memory operation in flight)
        __builtin_amdgcn_sched_barrier(0);
        float rs = 0.f;
        uint32_t pk[TNe][2];
#pragma unroll
        for (int j = 0; j < TNe; ++j) {
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            v[r] = act_static<ACT>(acc_read(acc[i][j][r]) + bc[j][r]);
            if (want_sq && ok[j]) rs += v[r] * v[r];
          }
          pk[j][0] = pack_bf16x2(v[0], v[1]);
          pk[j][1] = pack_bf16x2(v[2], v[3]);
        }
        if (want_sq) {
          // the row's four lanes (fc), then (below) the wave columns in order
          rs += __int_as_float(xor_lane<16>(__float_as_int(rs)));
          rs += __int_as_float(xor_lane<32>(__float_as_int(rs)));
          if (fc == 0) s_sq[sq_col][r0 + i * MF + fr] = rs;
        }
        if constexpr (NTS) {
#pragma unroll
          for (int p2 = 0; p2 < TNe / 4; ++p2) {
            // permlane16_swap(X, Y) trades X's rows 1, 3 for Y's rows 0, 2
            // (rows of 16 lanes): even rows end with [X, partner's X], odd rows
            // with [partner's Y, Y] -- 8 columns of the lane's row, at
            // colbase + 32 q, for q = 2 p2 (v[0]) and 2 p2 + 1 (v[1])
            u32x4_t v[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int q = 2 * p2 + h;
              const auto w0 = __builtin_amdgcn_permlane16_swap(pk[2 * q][0], pk[2 * q + 1][0], false, false);
              const auto w1 = __builtin_amdgcn_permlane16_swap(pk[2 * q][1], pk[2 * q + 1][1], false, false);
              v[h] = u32x4_t{w0[0], w1[0], w0[1], w1[1]};
            }
            // Whole 128-byte lines: lanes fr and fr ^ 8 (row_ror:8 inside each
            // 16-lane row) trade pieces so that the first store holds rows
            // 0 .. 7 of the slice and the second rows 8 .. 15, each row's 64
            // columns 64 p2 .. + 63 from eight lanes (fr < 8: q = 2 p2, fr >= 8:
            // q = 2 p2 + 1).  The bank masks pick the lanes that take their
            // partner's piece (banks 2, 3 are lanes 8 .. 15 of a row).
            u32x4_t s[2];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              s[0][d] = __builtin_amdgcn_update_dpp(v[0][d], v[1][d], 0x128, 0xF, 0xC, false);
              s[1][d] = __builtin_amdgcn_update_dpp(v[1][d], v[0][d], 0x128, 0xF, 0x3, false);
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              // formed here: the empty asm keeps the offset from being computed
              // (and kept live) ahead of time
              uint32_t off = lane_off;
              asm volatile("" : "+v"(off));
              off += (uint32_t)(((i * MF + 8 * h) * N + 64 * p2) * 2);
              // Non-temporal: the output is not read again in this pass.
              if (lane_row + 8 * h < cur_t.M - i * MF && n0 + c0 + colbase + 64 * p2 < N)
                __builtin_nontemporal_store(s[h], (u32x4_t*)(cbase + off));
            }
          }
        } else {
#pragma unroll
          for (int q = 0; q < TNe / 2; ++q) {
            // the 8 columns of the lane's row at colbase + 32 q (as above)
            const auto w0 = __builtin_amdgcn_permlane16_swap(pk[2 * q][0], pk[2 * q + 1][0], false, false);
            const auto w1 = __builtin_amdgcn_permlane16_swap(pk[2 * q][1], pk[2 * q + 1][1], false, false);
            vec16 val;
            val.w[0] = w0[0];
            val.w[1] = w1[0];
            val.w[2] = w0[1];
            val.w[3] = w1[1];
            uint32_t off = lane_off;
            asm volatile("" : "+v"(off));
            off += (uint32_t)((i * MF * N + 32 * q) * 2);
            if (lane_row < cur_t.M - i * MF && n0 + c0 + colbase + 32 * q < N) *(vec16*)(cbase + off) = val;
          }
        }
      }
    };
    const int cur_mode = tile_mode(cur_t.M, cur_t.nt);  // uniform
    if (cur_mode == M_HALF_H) {
      epilogue(std::integral_constant<int, M_HALF_H>{});
    } else if (cur_mode == M_HALF_W) {
      if constexpr (kHalfW) epilogue(std::integral_constant<int, M_HALF_W>{});
    } else {
      epilogue(std::integral_constant<int, M_FULL>{});
    }
    // every wave has read this tile's bias and written its row sums: the
    // next tile's bias may land, the sums may be added.  LDS only, so the
    // barrier waits for LDS accesses alone (__syncthreads would also wait
    // for every load and store in flight: the next tile's first stages and
    // this tile's output)
    slab_barrier();
    if (want_sq) {
      // the wave columns' partial sums in column order (half-height tiles
      // add four, so their sums round differently from a full tile's; a
      // half-width tile has one, the full tile's first, its second being
      // past N).  The empty asm keeps the row's LDS addresses from being
      // formed at kernel start and kept (spilled) through the K loop.
      int m0 = tid;
      asm volatile("" : "+v"(m0));
      if (cur_mode == M_HALF_H)
        for (int m = m0; m < cur_t.M; m += C::NT)
          p.sq_part[(cur_t.row0 + m) * (int64_t)n_tiles + cur_t.nt] = ((s_sq[0][m] + s_sq[1][m]) + s_sq[2][m]) + s_sq[3][m];
      else if (cur_mode == M_HALF_W)
        for (int m = m0; m < cur_t.M; m += C::NT)
          p.sq_part[(cur_t.row0 + m) * (int64_t)n_tiles + cur_t.nt] = s_sq[0][m];
      else
        for (int m = m0; m < cur_t.M; m += C::NT)
          p.sq_part[(cur_t.row0 + m) * (int64_t)n_tiles + cur_t.nt] = s_sq[0][m] + s_sq[1][m];
    }
    if (tl.M < 0) break;  // uniform
    load_bias(tl);
  }
}

template <int SUB>
static hipError_t launch_persist(const GemmArgs& a, hipStream_t st) {
  const int64_t rows = a.group_offset ? a.max_rows : a.dense_M;
  if (rows <= 0) return hipSuccess;
  const int64_t mt = (rows + 255) / 256 + (a.group_offset ? a.G : 0);
  const int64_t bound = grid_blocks(mt, (a.N + 255) / 256);
  const int64_t blocks = bound < kCus ? bound : kCus;  // a multiple of 8 either way
  // Outputs beyond the 256 MB Infinity Cache (the large layer's 0.8 and
  // 2.1 GB) go out as whole non-temporal lines; smaller ones (read back by
  // the next pass from that cache) as plain row pieces, which measured 2-3 %
  // faster there (64-expert layers, outputs of 33-201 MB).
  const bool nts = rows * (int64_t)a.N * 2 > ((int64_t)256 << 20);
#define MOE_PERSIST(ACTV)                                                                                         \
  do {                                                                                                           \
    if (nts) hipLaunchKernelGGL((gemm_bf16_persist_kernel<SUB, ACTV, true>), dim3((unsigned)blocks), dim3(256), 0, st, a);  \
    else hipLaunchKernelGGL((gemm_bf16_persist_kernel<SUB, ACTV, false>), dim3((unsigned)blocks), dim3(256), 0, st, a); \
  } while (0)
  switch (a.act) {
    case ACT_RELU: MOE_PERSIST(ACT_RELU); break;
    case ACT_GELU: MOE_PERSIST(ACT_GELU); break;
    case ACT_SWISH: MOE_PERSIST(ACT_SWISH); break;
    default: MOE_PERSIST(-1); break;
  }
#undef MOE_PERSIST
  return hipGetLastError();
}

bool gemm_persist_supported(const GemmArgs& a) {
  const int64_t rows = a.group_offset ? a.max_rows : a.dense_M;
  const int64_t list = ((rows + 255) / 256 + (a.group_offset ? a.G : 0)) * ((a.N + 255) / 256);
  return a.S <= 1 && !a.out_f32 && a.K % 32 == 0 && a.K >= 64 && a.N % 8 == 0 &&
         (a.group_offset == nullptr || a.G <= 256) && list < ((int64_t)1 << 30) &&
         (int64_t)a.N * a.K < ((int64_t)1 << 31) && rows < ((int64_t)1 << 31);
}

hipError_t launch_gemm_bf16_persist(const GemmArgs& a, hipStream_t st) {
  if (!gemm_persist_supported(a)) return hipErrorInvalidValue;
  return a.K % 64 == 0 ? launch_persist<2>(a, st) : launch_persist<1>(a, st);
}

}  // namespace moe
