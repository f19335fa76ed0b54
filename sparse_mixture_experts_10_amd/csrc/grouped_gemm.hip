// Grouped GEMM over ragged per-expert row ranges, used twice per expert FFN.
//
// Each expert is a two-layer MLP w1/b1 -> activation -> w2/b2 (page "Code
// Walkthrough -- SER", the gating / routing path); over all the rows the
// dispatch packed for expert g this is
//   pass 1:  H = act(X_g W1_g^T + b1_g)        (N = F,     K = d)
//   pass 2:  Y = H W2_g^T + b2_g               (N = d_out, K = F)
// with W in (out x in) layout, so both operands are K-contiguous.
//
// bf16 path: CDNA4 MFMA v_mfma_f32_16x16x32_bf16, fp32 accumulation, fp32
// epilogue (bias, activation, optional per-row sum of squares of the
// activation before rounding), one round-to-nearest-even to bf16.
// Tile 128 x 128 x 64, 256 threads = 4 waves in 2 x 2, each wave 64 x 64 as
// 4 x 4 MFMA tiles.  Global -> registers -> LDS, two LDS buffers (one barrier
// per K step), rows padded by 16 bytes so the MFMA operand reads are
// bank-conflict free.  The output tile is staged through LDS so every global
// store is a full 16-byte vector.
//
// Ragged groups: the 1-D grid is sized from a host bound on the row count;
// each block finds its (group, row tile, N tile) from the device-side group
// offsets with a wave-wide prefix scan, and blocks past the last tile exit at
// once.  The host never reads the per-expert counts.  Tiles are dealt to the
// 8 XCDs in contiguous bands (see find_tile) for L2 locality.

#include "common.h"
#include "internal.h"
#include "gemm_tiles.h"

namespace moe {

namespace {

__device__ __forceinline__ float bias_at(const bf16_t* bias, int g, int S, int N, int n) {
  if (bias == nullptr) return 0.f;
  if (S <= 1) return bf16_to_f32(bias[(int64_t)g * N + n]);
  float s = 0.f;
  for (int q = 0; q < S; ++q) s += bf16_to_f32(bias[(int64_t)q * N + n]);
  return s;
}

__device__ __forceinline__ float bias_at(const float* bias, int g, int S, int N, int n) {
  if (bias == nullptr) return 0.f;
  if (S <= 1) return bias[(int64_t)g * N + n];
  float s = 0.f;
  for (int q = 0; q < S; ++q) s += bias[(int64_t)q * N + n];
  return s;
}

}  // namespace

// ---------------------------------------------------------------------------
// bf16 MFMA path
// ---------------------------------------------------------------------------
constexpr int BM = kGemmBM, BN = kGemmBN, BK = 64, LDK = BK + 8, LDC = BN + 8;

template <bool SEG>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * (BM + BN) * LDK];
  __shared__ int s_info[4];
  __shared__ float s_sq[2][BM];

  const int n_tiles = (p.N + BN - 1) / BN;
  const Tile tl = find_tile<BM>(p.group_offset, p.G, p.dense_M, p.max_rows, n_tiles, s_info, p.n_major);
  if (tl.M <= 0) return;  // uniform

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int N = p.N, K = p.K;
  const int n0 = tl.nt * BN;
  const bf16_t* A = (const bf16_t*)p.A;
  const bf16_t* B = (const bf16_t*)p.B;
  const int64_t Bg = SEG ? 0 : (int64_t)tl.g * N * K;

  // per-thread load slots: 4 A vectors and 4 B vectors per K step
  int64_t a_off[4];
  int64_t b_off[4];
  int l_row[4], l_cv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int v = tid + 256 * i;
    l_row[i] = v >> 3;
    l_cv[i] = v & 7;
    const int ar = l_row[i] < tl.M ? l_row[i] : tl.M - 1;
    const int64_t arow = p.a_rows ? (int64_t)p.a_rows[tl.row0 + ar] : tl.row0 + ar;
    a_off[i] = arow * (int64_t)K;
    const int bn = (n0 + l_row[i] < N) ? n0 + l_row[i] : N - 1;
    b_off[i] = SEG ? (int64_t)bn * p.Kseg : Bg + (int64_t)bn * K;
  }

  vec16 ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int col = k0 + l_cv[i] * 8;
      if (col < K) {
        ra[i] = *(const vec16*)(A + a_off[i] + col);
        if (SEG) {
          const int s = col / p.Kseg;
          const int kk = col - s * p.Kseg;
          rb[i] = *(const vec16*)(B + (int64_t)s * N * p.Kseg + b_off[i] + kk);
        } else {
          rb[i] = *(const vec16*)(B + b_off[i] + col);
        }
      } else {
        ra[i] = vec16{{0u, 0u, 0u, 0u}};
        rb[i] = vec16{{0u, 0u, 0u, 0u}};
      }
    }
  };
  auto sstore = [&](int buf) {
    bf16_t* As = smem + buf * (BM + BN) * LDK;
    bf16_t* Bs = As + BM * LDK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *(vec16*)(As + l_row[i] * LDK + l_cv[i] * 8) = ra[i];
      *(vec16*)(Bs + l_row[i] * LDK + l_cv[i] * 8) = rb[i];
    }
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = (K + BK - 1) / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  const int fr = lane & 15;
  const int fk = (lane >> 4) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) gload((kt + 1) * BK);
    const bf16_t* As = smem + (kt & 1) * (BM + BN) * LDK;
    const bf16_t* Bs = As + BM * LDK;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      bf16x8_t a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *(const bf16x8_t*)(As + (wm * 64 + i * 16 + fr) * LDK + kk + fk);
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = *(const bf16x8_t*)(Bs + (wn * 64 + j * 16 + fr) * LDK + kk + fk);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore((kt + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds C[wm*64 + i*16 + 4*(lane>>4) + r][wn*64 + j*16 + (lane&15)] ----
  bf16_t* Cs = smem;
  const bf16_t* bias = (const bf16_t*)p.bias;
  float bcol[4];
  bool ncol_ok[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + wn * 64 + j * 16 + fr;
    ncol_ok[j] = n < N;
    bcol[j] = ncol_ok[j] ? bias_at(bias, tl.g, SEG ? p.S : 1, N, n) : 0.f;
  }
  const bool want_sq = p.sq_part != nullptr;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = acc[i][j][r] + bcol[j];
        if (p.act >= 0) v = apply_act(p.act, v);
        if (ncol_ok[j]) rs[r] += v * v;
        const int m = wm * 64 + i * 16 + (lane >> 4) * 4 + r;
        const int n = wn * 64 + j * 16 + fr;
        Cs[m * LDC + n] = f32_to_bf16(v);
      }
    }
    if (want_sq) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float s = rs[r];
        s += __shfl_xor(s, 1, 64);
        s += __shfl_xor(s, 2, 64);
        s += __shfl_xor(s, 4, 64);
        s += __shfl_xor(s, 8, 64);
        if (fr == 0) s_sq[wn][wm * 64 + i * 16 + (lane >> 4) * 4 + r] = s;
      }
    }
  }
  __syncthreads();
  bf16_t* C = (bf16_t*)p.C;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int v = tid + 256 * i;
    const int r = v >> 4, cv = v & 15;
    const int n = n0 + cv * 8;
    if (r < tl.M && n < N)
      *(vec16*)(C + (tl.row0 + r) * (int64_t)N + n) = *(const vec16*)(Cs + r * LDC + cv * 8);
  }
  if (want_sq && tid < tl.M)
    p.sq_part[(tl.row0 + tid) * (int64_t)n_tiles + tl.nt] = s_sq[0][tid] + s_sq[1][tid];
}

// Tile choice from host-side bounds (the row counts stay on the device):
//   0    register-staged kernel (K not a multiple of 32)
//   64   128 x 64 (narrow N)
//   128  128 x 128, eight waves
//   144  144 x 128, two blocks per CU (twelve waves and 64-wide K stages, or
//        six waves and 32-wide stages when K is not a multiple of 64)
//   145  144 x 128, twelve waves, 64-wide K stages, one block per CU
//   257  128 x 256, eight waves, two blocks per CU: many waves of tiles,
//        wide N, K < 2048
//   259  128 x 128, eight waves, 64-wide K stages and a 4-stage ring, one
//        block per CU: many waves of tiles, K >= 2048
//        (measured on MI355X on the switch workload's passes, groups of at
//        most 256 rows: up, K 1024, 174 -> 156 us; down, K 4096, 174 -> 146 us)
//   256  256 x 128, eight waves: many tiles and groups of >= 512 rows
//   513  256 x 256, eight waves in two ping-pong groups, 32-wide K stages in
//        a 4-stage ring: groups of >= 512 rows over four or more waves of
//        tiles, or groups of >= 1536 rows (the weight tiles are re-read from
//        L2 the fewest times; measured on MI355X against the 64-wide 2-stage
//        ring it replaces: the two shared experts of the fine-grained layer,
//        d 2048, F 1408, 8192 rows, 218 -> 186 us); when K has one segment
//        and the output is bf16, the persistent four-wave kernel instead
//        (gemm_bf16_persist.hip; 128 groups of 2048 rows at d 4096, F 1536:
//        up 1047 -> 1091, down 1034 -> 1109 TFLOP/s; with its half-width
//        mode also N = 1408, the fine-grained up pass, 380 -> 345 us)
// Between 128 and 144 rows, for passes of at most four waves of 128-row tiles,
// the one that puts the fewest rows on the busiest CU wins, with every group
// assumed to hold its mean share plus 8 % (routing imbalance).  A group of up to 1152 rows then takes eight 144-row tiles
// instead of nine 128-row ones: on the 8-expert, 8192-row passes the tile
// count drops to a whole number of waves over the CUs (measured on MI355X:
// down pass 22 -> 17.7 us; the 64-wide-stage variant when one tile per CU
// covers the pass).
static int bf16_tile(const GemmArgs& a) {
  if (!gemm_v2_supported(a)) return 0;
  if (a.N <= 64) return 64;
  const int64_t rows = a.group_offset ? a.max_rows : a.dense_M;
  const int64_t per_group = a.group_offset ? rows / a.G : rows;
  const int64_t groups = a.group_offset ? a.G : 1;
  const int64_t est = a.group_offset ? (per_group * 108 + 99) / 100 : rows;
  // 256 x 256 tiles (32-wide 4-stage ring, ping-pong waves) for several
  // waves of tiles or for groups of 1536 rows and more
  const int64_t t256 = groups * ((est + 255) / 256) * ((a.N + 255) / 256);
  if (a.N >= 256 && per_group >= 512 && t256 >= 4 * kCus) return 513;
  if (a.N >= 512 && per_group >= 1536) return 513;
  const int64_t big = ((rows + 255) / 256 + (a.group_offset ? a.G : 0)) * ((a.N + 127) / 128);
  if (big >= 1024 && per_group >= 512) return 256;
  const int64_t nt = (a.N + 127) / 128;
  const int64_t t128 = groups * ((est + 127) / 128) * nt;
  const int64_t t144 = groups * ((est + 143) / 144) * nt;
  // over several waves of tiles the last wave's share is small and 128 rows
  // waste fewer rows on partly filled groups (capacity-capped ones sit exactly
  // on 128-row multiples).  A long K loop takes 64-wide stages and a deep
  // ring; wide N with a short K loop takes 128 x 256 tiles (64 x 64 a wave).
  if (t128 > 4 * kCus) {
    if (a.K >= 2048 && gemm_v2_wide_k(a)) return 259;
    if (a.N >= 512) return 257;
    return 128;
  }
  const int64_t cost128 = (t128 + kCus - 1) / kCus * 128;
  const int64_t cost144 = (t144 + kCus - 1) / kCus * 144;
  if (cost144 < cost128) return (t144 <= kCus && gemm_v2_wide_k(a)) ? 145 : 144;
  return 128;
}

int gemm_bf16_n_tiles(const GemmArgs& a) {
  const int t = bf16_tile(a);
  const int bn = t == 64 ? 64 : (t == 513 || t == 257) ? 256 : 128;
  return (a.N + bn - 1) / bn;
}

// Tile order inside a group: a group's weight tile is read once per row tile,
// its A rows once per N tile.  When the weights outweigh the rows (N G >
// rows: small groups, wide layers) the N-major order runs a weight tile's row
// tiles back to back, so the repeats hit L2.
static bool gemm_n_major(const GemmArgs& a) {
  return a.group_offset != nullptr && (int64_t)a.N * a.G > a.max_rows;
}

hipError_t launch_gemm_bf16(const GemmArgs& a0, hipStream_t st) {
  GemmArgs a = a0;
  a.n_major = gemm_n_major(a);
  const int t = bf16_tile(a);
  // The persistent 256 x 256 kernel takes the N-major order for every
  // grouped pass: with 32 blocks of an XCD walking neighbouring tiles, a
  // round then spans few weight tiles over all of an expert's row tiles
  // (measured on MI355X, 128 experts of 2048 rows at d 4096, F 1536: up
  // pass 2999 -> 2956 us; the down pass is N-major by the rule above; on the
  // 8-expert default passes, which take other kernels, N-major measured
  // 1 % slower).
  if (t == 513 && a.group_offset != nullptr && gemm_persist_supported(a)) a.n_major = true;
  if (t) return launch_gemm_bf16_v2(a, t, st);
  return launch_gemm_bf16_v1(a, st);
}

hipError_t launch_gemm_bf16_v1(const GemmArgs& a, hipStream_t st) {
  const int64_t rows = a.group_offset ? a.max_rows : a.dense_M;
  const int64_t mt = (rows + BM - 1) / BM + (a.group_offset ? a.G : 0);
  if (rows <= 0) return hipSuccess;
  const dim3 grid((unsigned)grid_blocks(mt, (a.N + BN - 1) / BN));
  if (a.S > 1)
    hipLaunchKernelGGL(gemm_bf16_kernel<true>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(gemm_bf16_kernel<false>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp32 path (plain FMA; for fp32 layers)
// ---------------------------------------------------------------------------
constexpr int FBM = kGemmF32BM, FBN = kGemmF32BN, FBK = 16;

__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs p) {
  __shared__ float As[FBK][FBM + 4];
  __shared__ float Bs[FBK][FBN + 4];
  __shared__ int s_info[4];

  const int n_tiles = (p.N + FBN - 1) / FBN;
  const Tile tl = find_tile<FBM>(p.group_offset, p.G, p.dense_M, p.max_rows, n_tiles, s_info, p.n_major);
  if (tl.M <= 0) return;

  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int N = p.N, K = p.K;
  const int n0 = tl.nt * FBN;
  const float* A = (const float*)p.A;
  const float* B = (const float*)p.B;
  const bool seg = p.S > 1;

  const int lr = tid >> 2, lc = (tid & 3) * 4;
  const int ar = lr < tl.M ? lr : tl.M - 1;
  const float* arow = A + (p.a_rows ? (int64_t)p.a_rows[tl.row0 + ar] : tl.row0 + ar) * (int64_t)K;
  const int bn = (n0 + lr < N) ? n0 + lr : N - 1;

  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += FBK) {
    const int col = k0 + lc;
    float4 av = make_float4(0.f, 0.f, 0.f, 0.f), bv = av;
    if (col < K) {
      av = *(const float4*)(arow + col);
      if (seg) {
        const int s = col / p.Kseg;
        bv = *(const float4*)(B + ((int64_t)s * N + bn) * p.Kseg + (col - s * p.Kseg));
      } else {
        bv = *(const float4*)(B + ((int64_t)tl.g * N + bn) * K + col);
      }
    }
    As[lc + 0][lr] = av.x; As[lc + 1][lr] = av.y; As[lc + 2][lr] = av.z; As[lc + 3][lr] = av.w;
    Bs[lc + 0][lr] = bv.x; Bs[lc + 1][lr] = bv.y; Bs[lc + 2][lr] = bv.z; Bs[lc + 3][lr] = bv.w;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FBK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }

  const float* bias = (const float*)p.bias;
  float* C = (float*)p.C;
  const bool want_sq = p.sq_part != nullptr;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = ty * 4 + i;
    float v[4];
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      v[j] = acc[i][j] + ((n < N) ? bias_at(bias, tl.g, seg ? p.S : 1, N, n) : 0.f);
      if (p.act >= 0) v[j] = apply_act(p.act, v[j]);
      if (n < N) rs += v[j] * v[j];
    }
    if (r < tl.M && n0 + tx * 4 < N)
      *(float4*)(C + (tl.row0 + r) * (int64_t)N + n0 + tx * 4) = make_float4(v[0], v[1], v[2], v[3]);
    if (want_sq) {
      rs += __shfl_xor(rs, 1, 64);
      rs += __shfl_xor(rs, 2, 64);
      rs += __shfl_xor(rs, 4, 64);
      rs += __shfl_xor(rs, 8, 64);
      if (tx == 0 && r < tl.M) p.sq_part[(tl.row0 + r) * (int64_t)n_tiles + tl.nt] = rs;
    }
  }
}

hipError_t launch_gemm_f32(const GemmArgs& a, hipStream_t st) {
  const int64_t rows = a.group_offset ? a.max_rows : a.dense_M;
  const int64_t mt = (rows + FBM - 1) / FBM + (a.group_offset ? a.G : 0);
  if (rows <= 0) return hipSuccess;
  const dim3 grid((unsigned)grid_blocks(mt, (a.N + FBN - 1) / FBN));
  hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

// sq[r] = sum over N tiles of the per-tile partial sums, in tile order.
__global__ void sq_reduce_kernel(const float* __restrict__ part, int n_tiles,
                                 const int32_t* __restrict__ goff, int G, int64_t max_rows,
                                 float* __restrict__ sq) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t rows = goff[G] < max_rows ? goff[G] : max_rows;
  if (r >= rows) return;
  float s = 0.f;
  for (int q = 0; q < n_tiles; ++q) s += part[r * n_tiles + q];
  sq[r] = s;
}

hipError_t launch_sq_reduce(const float* sq_part, int n_tiles, const int32_t* group_offset, int G,
                            int64_t max_rows, float* sq, hipStream_t st) {
  if (max_rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(sq_reduce_kernel, dim3((unsigned)((max_rows + 255) / 256)), dim3(256), 0, st,
                     sq_part, n_tiles, group_offset, G, max_rows, sq);
  return hipGetLastError();
}

}  // namespace moe
