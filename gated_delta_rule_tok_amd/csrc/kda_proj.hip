// kda_proj.hip -- the low-rank gate and beta projections upstream of the KDA
// forward, as two skinny GEMMs for few tokens (a decode step).
//
// The PR #55426 report ("Fix KDA projection overlap on Hopper",
// "Implementation breakdown" items 1-3 and "Key source snippets") runs them as
// skinny N and K GEMMs with bf16 operands and fp32 accumulation:
//   P = hidden [M, K] x W_ab^T        W_ab [128 + n_beta, K]: the gate's first
//                                     factor (F_A, rank 128) and the beta rows
//   G = P[:, :128] x W_b^T            W_b [H 128, 128]: the gate's second factor
// and its test shapes are K = 7168, 144 = 128 + 16 rows in W_ab, W_b of
// 1536 x 128, and 2-14 tokens.  P and G are rounded to bf16 (round to nearest
// even): G is the forward's raw gate input g [M, H, 128] and P's beta columns
// its raw beta logits (a strided column slice, token stride 128 + n_beta).
//
// gfx950 plan.  With few tokens the first product is a read of W_ab (2 MB at
// the test shape) that only the whole machine reads fast, so K is split over
// workgroups: workgroup (K slice of 1024, 16 rows of W_ab, 16 tokens) has four
// waves on 256-wide quarters of the slice, each forming a 16 x 16 partial with
// 16x16x32 bf16 MFMAs (each lane reads 16 contiguous bytes of a W_ab row and of
// a hidden row); the quarters are added in LDS in wave order and the slice's
// partial goes to the workspace.  No workgroup waits for another: handing
// partials between workgroups inside one launch would need device-scope
// release / acquire, which on this chip writes back and invalidates a whole
// XCD's L2 per workgroup.  The second launch starts after the first has ended
// (the stream orders them): each of its workgroups adds the slices of P's
// first 128 columns in slice order (so the result does not depend on the
// schedule), rounds them to bf16 into LDS, writes its share of P, and forms
// four 16 x 16 tiles of G from LDS against W_b.
#include <algorithm>

#include "kda_mfma.h"

namespace kda {
namespace {

constexpr int kAbWaves = 4;                 // waves per workgroup, first product
constexpr int kWaveK = 256;                 // K per wave of the first product
constexpr int kSliceK = kAbWaves * kWaveK;  // K per workgroup of the first product
constexpr int kWaves = 4;                   // waves per workgroup, second launch
constexpr int kSumBatch = 16;               // partial loads in flight per thread
constexpr int kLdsPitch = kProjRank + 8;  // bf16 per LDS row of P (bank spread)

__device__ __forceinline__ bf16x8 load8(const uint16_t* base, bool ok) {
  // 16 contiguous bytes (8 bf16), or zeros outside the matrix
  if (!ok) return bf16x8{};
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(base));
}

// Partial tile (slice ks, row tile nt of W_ab, token tile mt): 256 floats,
// element (token 4 g + j, column c) at 16 c + 4 g + j.
__device__ __forceinline__ size_t part_index(const ProjParams& pp, int mt, int nt, int ks) {
  const int nsl = (pp.K + kSliceK - 1) / kSliceK;
  const int ntab = (pp.n_ab + 15) / 16;
  return ((size_t(mt) * ntab + nt) * nsl + ks) * 256;
}

// First product: workgroup (K slice, row tile of W_ab, token tile), 4 waves.
// The dispatcher hands workgroup B to XCD (B + o) mod 8, so index B = 8 r +
// x carries slice ks = 8 (r / (row tiles x token tiles)) + x: every
// workgroup of one K slice sits on one XCD and the slice of the hidden
// states is fetched into that XCD's L2 once (indices past the last slice
// exit).
__global__ __launch_bounds__(64 * kAbWaves) void proj_ab_kernel(ProjParams pp) {
  __shared__ f32x4 red[kAbWaves][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int ntab = (pp.n_ab + 15) / 16, nmt = (pp.M + 15) / 16;
  const int nsl = (pp.K + kSliceK - 1) / kSliceK;
  const int r = blockIdx.x >> 3, nt = r % ntab, mt = (r / ntab) % nmt;
  const int ks = 8 * (r / (ntab * nmt)) + (blockIdx.x & 7);
  if (ks >= nsl) return;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int m = mt * 16 + l16;          // A operand row (token)
  const int n = nt * 16 + l16;          // B operand column (row of W_ab)
  const int k0 = ks * kSliceK + w * kWaveK, k1 = min(k0 + kWaveK, pp.K);
  const bool mok = m < pp.M, nok = n < pp.n_ab;
  const uint16_t* arow = pp.hidden + size_t(mok ? m : 0) * pp.K;
  const uint16_t* brow = pp.w_ab + size_t(nok ? n : 0) * pp.K;
  // all of the quarter's loads first, then the products
  constexpr int kSteps = kWaveK / 32;
  bf16x8 a[kSteps], b[kSteps];
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const int k = k0 + 32 * s + 8 * g4;  // K % 8 == 0: k < k1 covers k + 8
    a[s] = load8(arow + k, mok && k < k1);
    b[s] = load8(brow + k, nok && k < k1);
  }
  f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kSteps; ++s) c = mfma32(a[s], b[s], c);
  red[w][lane] = c;
  __syncthreads();
  if (w != 0) return;
  f32x4 sum = red[0][lane];
#pragma unroll
  for (int i = 1; i < kAbWaves; ++i) sum += red[i][lane];
  float* part = pp.partials + part_index(pp, mt, nt, ks);
  *reinterpret_cast<f32x4*>(part + 16 * l16 + 4 * g4) = sum;
}

// Sums over the slices, in slice order, of NI float4s of partial tiles (item
// i at p[i], slice j 256 floats further on).  A batch of slices is loaded for
// every item before the first add -- one memory latency per batch -- and the
// loads are unconditional (indices past the last slice read the last slice
// again and are not added), so that no branch splits the batch.
template <int NI>
__device__ __forceinline__ void slice_sums(const float* const (&p)[NI], int nsl, f32x4 (&s)[NI]) {
  constexpr int kBatch = kSumBatch / NI;
  for (int i0 = 0; i0 < nsl; i0 += kBatch) {
    f32x4 v[NI][kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const size_t j = size_t(min(i0 + b, nsl - 1)) * 256;
#pragma unroll
      for (int i = 0; i < NI; ++i) v[i][b] = *reinterpret_cast<const f32x4*>(p[i] + j);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      s[i] = i0 == 0 ? v[i][0] : s[i] + v[i][0];
#pragma unroll
      for (int b = 1; b < kBatch; ++b) s[i] = i0 + b < nsl ? s[i] + v[i][b] : s[i];
    }
  }
}

// Second launch: workgroup (x, token tile mt), 4 waves, x up to the larger
// of G's column groups of 64 and W_ab's row tiles.  Workgroup x writes P's
// column tile x (if there is one) and G's column tiles 4x .. 4x + 3 (those
// that exist).  Index B = 8 (mt X + x) + c works when c = mt mod 8 (the
// others exit): a token tile's workgroups all sit on one XCD, which fetches
// its partial tiles once.
__global__ __launch_bounds__(256) void proj_out_kernel(ProjParams pp) {
  __shared__ __align__(16) uint16_t P[16][kLdsPitch];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int ntab = (pp.n_ab + 15) / 16;
  const int gx = max((pp.n_b / 16 + kWaves - 1) / kWaves, ntab);
  const int r = blockIdx.x >> 3, x = r % gx, mt = r / gx;
  if (int(blockIdx.x & 7) != (mt & 7)) return;
  const int gt = x * kWaves + w;  // this wave's G column tile
  const bool has_g = gt < pp.n_b / 16;
  const int l16 = lane & 15, g4 = lane >> 4;
  // this wave's W_b operand first: it does not depend on P, so its memory
  // latency overlaps the partials' below
  bf16x8 b[kProjRank / 32];
  const uint16_t* brow = pp.w_b + size_t(has_g ? gt * 16 + l16 : 0) * kProjRank;
#pragma unroll
  for (int s = 0; s < kProjRank / 32; ++s) b[s] = load8(brow + 32 * s + 8 * g4, has_g);
  const int nsl = (pp.K + kSliceK - 1) / kSliceK;
  // P[:, :128] of this token tile: 8 tiles x 64 float4, two per thread
  {
    const float* p[2];
    f32x4 s[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = t + 256 * r;
      p[r] = pp.partials + part_index(pp, mt, i >> 6, 0) + 4 * (i & 63);
    }
    slice_sums(p, nsl, s);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = t + 256 * r, nt = i >> 6, q = i & 63;
      const int col = nt * 16 + (q >> 2), row0 = 4 * (q & 3);
#pragma unroll
      for (int j = 0; j < 4; ++j) P[row0 + j][col] = f32_to_bf16(s[r][j]);
    }
  }
  // P's column tiles beyond the first 128 columns (the beta rows): reduced
  // and written straight from registers
  if (x >= kProjRank / 16 && x < ntab && t < 64) {
    const float* p[1] = {pp.partials + part_index(pp, mt, x, 0) + 4 * t};
    f32x4 sb[1];
    slice_sums(p, nsl, sb);
    const f32x4 s = sb[0];
    const int col = x * 16 + (t >> 2), row0 = mt * 16 + 4 * (t & 3);
    if (col < pp.n_ab) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (row0 + j < pp.M) pp.p_ab[size_t(row0 + j) * pp.n_ab + col] = f32_to_bf16(s[j]);
    }
  }
  __syncthreads();
  if (x < kProjRank / 16) {  // one of P's first 8 column tiles, from LDS
    const int r = t >> 4, c = t & 15, row = mt * 16 + r;
    if (row < pp.M) pp.p_ab[size_t(row) * pp.n_ab + x * 16 + c] = P[r][x * 16 + c];
  }
  if (!has_g) return;
  bf16x8 a[kProjRank / 32];
#pragma unroll
  for (int s = 0; s < kProjRank / 32; ++s)
    a[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&P[l16][32 * s + 8 * g4]));
  f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kProjRank / 32; ++s) c = mfma32(a[s], b[s], c);
  const int n = gt * 16 + l16;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = mt * 16 + 4 * g4 + j;
    if (row < pp.M) pp.g[size_t(row) * pp.n_b + n] = f32_to_bf16(c[j]);
  }
}

}  // namespace

size_t proj_workspace_bytes(int M, int K, int n_ab) {
  const size_t nmt = size_t((M + 15) / 16), ntab = size_t((n_ab + 15) / 16);
  const size_t nsl = size_t((K + kSliceK - 1) / kSliceK);
  return nmt * ntab * nsl * 256 * sizeof(float);  // one partial tile per workgroup
}

hipError_t launch_proj(const ProjParams& p, hipStream_t stream) {
  ProjParams arg = p;
  void* args[] = {&arg};
  const int nmt = (p.M + 15) / 16, ntab = (p.n_ab + 15) / 16;
  const int nsl = (p.K + kSliceK - 1) / kSliceK;
  const dim3 g1(8 * ((nsl + 7) / 8) * ntab * nmt);  // see proj_ab_kernel
  if (hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&proj_ab_kernel), g1,
                                     dim3(64 * kAbWaves), args, 0, stream);
      e != hipSuccess)
    return e;
  const int gx = std::max((p.n_b / 16 + kWaves - 1) / kWaves, ntab);
  const dim3 g2(8 * gx * nmt);  // see proj_out_kernel
  return hipLaunchKernel(reinterpret_cast<const void*>(&proj_out_kernel), g2, dim3(64 * kWaves),
                         args, 0, stream);
}

}  // namespace kda
