// kda_segment.hip -- the segment-parallel schedule for long sequences in
// calls with few (sequence, head) items, where one workgroup walking every
// chunk of a sequence leaves most of the machine idle (the low-parallelism
// regime of PR #52458's report, "Features and motivation"; the 1 x 16384
// workload of PR #55737's report, same section).
//
// The recurrence S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T
// is affine in the state, so a segment of tokens maps its entering state S to
// P S + R, with P the product of the segment's (I - b k k^T) Diag(a) factors
// (128 x 128) and R the state the segment reaches from zero.  Three steps:
//   1. summaries (the pipelined kernel in summary mode): every segment but a
//      sequence's last runs from [0 | I] over 256 columns, values [v | 0],
//      which gives [R | P] -- all segments at once;
//   2. this file's combine: S_0 = the initial state, S_{j+1} = P_j S_j + R_j,
//      serial over a sequence's segments but only 128 x 128 x 16 per step
//      and workgroup;
//   3. the pipelined kernel over all segments at once, each from its S_j,
//      writing the outputs, and the last one the final state.
// This file holds the table of segments and the combine.
#include <type_traits>

#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kPlanThreads = 1024;

__device__ __forceinline__ void seq_bounds(const SegParams& sp, int n, int& b, int& e) {
  b = min(max(sp.cu[n], 0), sp.T);
  e = min(max(sp.cu[n + 1], b), sp.T);
}

// Inclusive scan of one value per thread over the workgroup (Hillis-Steele
// in LDS); returns this thread's inclusive sum, *total the workgroup's.
__device__ int block_scan(int x, int* buf, int* total) {
  const int t = threadIdx.x;
  buf[t] = x;
  __syncthreads();
  for (int off = 1; off < kPlanThreads; off <<= 1) {
    const int y = t >= off ? buf[t - off] : 0;
    __syncthreads();
    buf[t] += y;
    __syncthreads();
  }
  const int r = buf[t];
  *total = buf[kPlanThreads - 1];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kPlanThreads) void seg_plan_kernel(SegParams sp) {
  __shared__ int buf[kPlanThreads];
  const int t = threadIdx.x;
  // segment counts and the first pseudo-sequence of every sequence
  int carry = 0;
  for (int base = 0; base < sp.N; base += kPlanThreads) {
    const int n = base + t;
    int cnt = 0;
    if (n < sp.N) {
      int b, e;
      seq_bounds(sp, n, b, e);
      cnt = max(1, (e - b + sp.L - 1) / sp.L);
    }
    int tot;
    const int incl = block_scan(cnt, buf, &tot);
    if (n < sp.N) {
      sp.first[n] = carry + incl - cnt;
      sp.count[n] = cnt;
    }
    carry += tot;
  }
  // Well-formed offsets give at most N + T / L segments (each sequence at
  // most 1 + floor(len / L), the lengths summing to at most T).  Offsets that
  // overlap can give more: then every sequence is one segment.
  const bool whole = carry > sp.M;
  const int used = whole ? sp.N : carry;
  __syncthreads();  // this thread's first / count writes above are its own
  for (int n = t; n < sp.N; n += kPlanThreads) {
    int b, e;
    seq_bounds(sp, n, b, e);
    const int f = whole ? n : sp.first[n], c = whole ? 1 : sp.count[n];
    if (whole) {
      sp.first[n] = f;
      sp.count[n] = 1;
    }
    for (int j = 0; j < c; ++j) {
      const int s0 = b + j * sp.L;
      const int e0 = j == c - 1 ? e : s0 + sp.L;
      *reinterpret_cast<int4*>(sp.table + 4 * size_t(f + j)) = int4{n, s0, e0, j == c - 1 ? 1 : 0};
    }
  }
  for (int m = used + t; m < sp.M; m += kPlanThreads)
    *reinterpret_cast<int4*>(sp.table + 4 * size_t(m)) = int4{-1, 0, 0, 0};
}

constexpr int kCombWaves = 8;  // one 16-row tile of the 128 rows each
constexpr int kCombThreads = 64 * kCombWaves;
constexpr int kPad = 4;  // floats of padding per LDS row

typedef float f32x4 __attribute__((ext_vector_type(4)));

// fp32 16x16x4 MFMA: lane l holds A[l % 16][l / 16] and B[l / 16][l % 16];
// the accumulator's element j is D[4 (l / 16) + j][l % 16].
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Workgroup (sequence n, head h, columns 16 cb .. 16 cb + 15), eight waves;
// wave w forms rows 16 w .. 16 w + 15 of each step's P S + R as one 16 x 16
// accumulator tile, in fp32 MFMAs over the 128 keys.  P's rows go straight
// from memory into the A operands (each lane reads 16-byte pieces of its
// row, the four lanes of a row adjacent ones; the key order inside the sum
// is the same permutation on both sides) and are fetched two steps ahead
// with R, since one step's products are shorter than a round trip to
// memory; S comes from a transposed LDS tile as 16-byte rows.  The 8 column
// blocks of one (n, h) go to one XCD (workgroup indices 8 apart), so each P
// is fetched into that XCD's L2 once.
__global__ __launch_bounds__(kCombThreads) void seg_combine_kernel(SegParams sp) {
  __shared__ __align__(16) float St[16][kD + kPad];  // St[column][key]
  const int B = blockIdx.x, xcd = B & 7, k = B >> 3;
  const int item = (k >> 3) * 8 + xcd, cb = k & 7;
  if (item >= sp.N * sp.H) return;
  const int n = item / sp.H, h = item % sp.H;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int col = 16 * cb + l16;
  const int row0 = 16 * w + 4 * g4;  // accumulator rows row0 .. row0 + 3
  const size_t DD = size_t(kD) * kD;
  // the state entering the current segment (accumulator layout), from the
  // initial state in fp32
  f32x4 s;
  const size_t ib = (size_t(n) * sp.H + h) * DD;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const size_t o = ib + size_t(row0 + j) * kD + col;
    s[j] = !sp.s0 ? 0.f
           : sp.s0_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(sp.s0)[o])
                        : static_cast<const float*>(sp.s0)[o];
  }
  const int f = sp.first[n], cnt = sp.count[n];
  // Operands of a step in a ring of three register sets: P[16 w + l16][16 q
  // + 4 g4 .. + 3] (q = 0..7; the four lanes of a row read 64 contiguous
  // bytes per load, one cache line per row and pair of loads) as A
  // operands, R in the accumulator layout.
  // Step j (segment f + j, j <= cnt - 2) uses set j % 3, fetched at the top
  // of step j - 2.
  float4 pb[3][8];
  f32x4 rb[3];
  auto fetch = [&](auto bi, int m) {
    constexpr int b = decltype(bi)::value;
    const float* R = sp.summ + (size_t(m) * sp.H + h) * 2 * DD;
    const float* Pm = R + DD;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      pb[b][q] = *reinterpret_cast<const float4*>(Pm + size_t(16 * w + l16) * kD + 16 * q + 4 * g4);
#pragma unroll
    for (int j = 0; j < 4; ++j) rb[b][j] = R[size_t(row0 + j) * kD + col];
  };
  auto store_start = [&](int m) {
    const size_t sb = (size_t(m) * sp.H + h) * DD;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) sp.starts[sb + size_t(row0 + jj) * kD + col] = s[jj];
  };
  // one step: the state entering segment f + j + 1; false past the last
  auto step = [&](auto bi, int j) -> bool {
    constexpr int b = decltype(bi)::value;
    if (j >= cnt - 1) return false;
    // the operands of step j + 2, into the set step j - 1 used; unconditional
    // (clamped to this sequence's last segment, whose slot is in the area and
    // whose values go unused), so every path issues the same memory
    // operations and the compiler's wait before the products below stays the
    // minimal one
    fetch(std::integral_constant<int, (b + 2) % 3>{}, f + min(j + 2, cnt - 1));
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) St[l16][row0 + jj] = s[jj];  // S, transposed
    f32x4 acc = rb[b];
    __syncthreads();
    // B operands S[16 q + 4 g4 + e][col]: the same key order as the A side
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float4 sv = *reinterpret_cast<const float4*>(&St[l16][16 * q + 4 * g4]);
      acc = mfma_f32(pb[b][q].x, sv.x, acc);
      acc = mfma_f32(pb[b][q].y, sv.y, acc);
      acc = mfma_f32(pb[b][q].z, sv.z, acc);
      acc = mfma_f32(pb[b][q].w, sv.w, acc);
    }
    s = acc;
    store_start(f + j + 1);
    __syncthreads();  // St is rewritten next step
    return true;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  store_start(f);  // first: the initial state's loads are then complete before the fetches
  fetch(I0{}, f);
  fetch(I1{}, f + min(1, cnt - 1));
  for (int j = 0;; j += 3) {
    if (!step(I0{}, j)) break;
    if (!step(I1{}, j + 1)) break;
    if (!step(I2{}, j + 2)) break;
  }
}

}  // namespace

hipError_t launch_seg_plan(const SegParams& sp, hipStream_t stream) {
  SegParams arg = sp;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&seg_plan_kernel), dim3(1), dim3(kPlanThreads),
                         args, 0, stream);
}

hipError_t launch_seg_combine(const SegParams& sp, hipStream_t stream) {
  SegParams arg = sp;
  void* args[] = {&arg};
  const int items = (sp.N * sp.H + 7) / 8 * 8;
  return hipLaunchKernel(reinterpret_cast<const void*>(&seg_combine_kernel), dim3(items * 8),
                         dim3(kCombThreads), args, 0, stream);
}

}  // namespace kda
