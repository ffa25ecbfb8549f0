// kda_recurrent.hip -- token-serial KDA forward in fp32 on the vector ALUs.
//
// One workgroup (4 waves) per (sequence, head, value slice).  The slice of the
// state, 128 key rows x VS value columns in fp32, lives in registers: each lane
// owns one value column and R = VS/2 consecutive key rows, and the lanes of a
// wave that share a column are the RG = 256/VS row groups.  Per token:
//     S <- Diag(a) S;  p = S^T k;  r = S^T (scale q)          (one sweep)
//     d = beta (v - p);  S <- S + k d^T;  o = r + (k . scale q) d
// which is the gated delta rule S_t = (I - b k k^T) Diag(a) S_{t-1} + b k v^T,
// o_t = scale S_t^T q_t with the rank-1 product expanded (the operation of
// vLLM PR #55737's report, "Features and motivation").  Column sums over the
// key rows reduce across the RG lanes of a column with cross-lane shuffles, in
// an order that does not depend on VS.
//
// Tokens are taken in blocks of kTB: the four waves first L2-normalise q and k,
// evaluate the bounded gate a = exp(lb * sigmoid(exp(A_log) (g + dt_bias))) and
// beta = sigmoid(logit) for the block (one token per wave at a time, two
// channels per lane) into LDS, then every lane walks the block token by token.
//
// Value columns never mix, so any split of the value dimension gives
// bit-identical results.
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kThreads = 256;

// State row base of (sequence n, head h): the sequence's own state, or, in a
// speculative-decode step, the pool slot it starts from (-1: the zero state).
__device__ __forceinline__ int64_t start_slot(const Params& p, int n) {
  if (!p.sp_idx) return n;
  const int a = p.sp_acc[n];
  if (a < 1 || a > p.sp_stride) return -1;
  const int64_t s = p.sp_idx[int64_t(n) * p.sp_stride + a - 1];
  return (s >= 0 && s < p.sp_slots) ? s : -1;
}
// The slot that receives the state after token i of sequence n's step (-1: none).
__device__ __forceinline__ int64_t step_slot(const Params& p, int n, int i) {
  if (i >= p.sp_stride) return -1;
  const int64_t s = p.sp_idx[int64_t(n) * p.sp_stride + i];
  return (s >= 0 && s < p.sp_slots) ? s : -1;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// kTB: tokens staged in LDS per step (32 for prefill; 4 for decode-sized
// sequences, which keeps the LDS block small so more workgroups stream their
// state at once)
template <int VS, int kTB>
__global__ __launch_bounds__(kThreads) void recurrent_kernel(Params p) {
  constexpr int CW = VS / 4;   // value columns per wave
  constexpr int RG = 64 / CW;  // row groups per wave
  constexpr int R = kD / RG;   // key rows per lane
  constexpr int GL = R / 8;    // 8-row reduction groups per lane
  static_assert(R % 8 == 0, "rows per lane must be a multiple of 8");

  __shared__ float s_q[kTB][kD];
  __shared__ float s_k[kTB][kD];
  __shared__ float s_a[kTB][kD];
  __shared__ uint16_t s_v[kTB][VS];  // raw bf16 (keeps the block under 64 KiB of LDS)
  __shared__ float s_beta[kTB];
  __shared__ float s_kq[kTB];

  const int slice = blockIdx.x % p.vsplit;
  const int rest = blockIdx.x / p.vsplit;
  const int h = rest % p.H;
  // sequence: from the order table, or the rank itself when there is none
  const int n = p.order ? p.order[rest / p.H] : rest / p.H;
  const int H = p.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane % CW, rg = lane / CW;
  const int jl = wave * CW + col;  // column inside the slice
  const int j = slice * VS + jl;   // value channel
  const int r0 = rg * R;           // first key row

  float S[R];
  const int64_t s0slot = start_slot(p, n);
  const size_t sbase = ((size_t)n * H + h) * kD * kD;
  const size_t s0base = ((size_t)max(s0slot, int64_t(0)) * H + h) * kD * kD;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const size_t idx = s0base + (size_t)(r0 + i) * kD + j;
    if (!p.s0 || s0slot < 0) S[i] = 0.f;
    else if (p.state_bf16) S[i] = bf16_to_f32(static_cast<const uint16_t*>(p.s0)[idx]);
    else S[i] = static_cast<const float*>(p.s0)[idx];
  }
  // the state after token i of a speculative-decode step, into its slot
  auto store_step = [&](int i) {
    const int64_t slot = step_slot(p, n, i);
    if (slot < 0) return;
    const size_t b = ((size_t)slot * H + h) * kD * kD;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const size_t idx = b + (size_t)(r0 + r) * kD + j;
      if (p.state_bf16) static_cast<uint16_t*>(p.sT)[idx] = f32_to_bf16(S[r]);
      else static_cast<float*>(p.sT)[idx] = S[r];
    }
  };

  const float eA = expf(p.A_log[h]);
  const float dtb0 = p.dt_bias[h * kD + 2 * lane];
  const float dtb1 = p.dt_bias[h * kD + 2 * lane + 1];
  // clamp the sequence to [0, T) so malformed offsets cannot leave the buffers
  // the bounds are uniform: scalar registers (else every buffer access with a
  // token offset in its scalar operand becomes a loop over lanes)
  const int bos = __builtin_amdgcn_readfirstlane(min(max(p.cu[n], 0), p.T));
  const int eos = __builtin_amdgcn_readfirstlane(min(max(p.cu[n + 1], bos), p.T));

  for (int t0 = bos; t0 < eos; t0 += kTB) {
    const int nt = min(kTB, eos - t0);
    for (int tt = wave; tt < nt; tt += 4) {
      const size_t t = size_t(t0 + tt);
      const uint32_t qp = reinterpret_cast<const uint32_t*>(p.q + t * p.ts_q + size_t(h) * p.hs_q)[lane];
      const uint32_t kp = reinterpret_cast<const uint32_t*>(p.k + t * p.ts_k + size_t(h) * p.hs_k)[lane];
      const uint32_t gp = reinterpret_cast<const uint32_t*>(p.g + t * p.ts_g + size_t(h) * p.hs_g)[lane];
      float q0 = bf16_lo(qp), q1 = bf16_hi(qp);
      float k0 = bf16_lo(kp), k1 = bf16_hi(kp);
      const float rq = rsqrtf(wave_sum(q0 * q0 + q1 * q1) + kNormEps) * p.scale;
      const float rk = rsqrtf(wave_sum(k0 * k0 + k1 * k1) + kNormEps);
      q0 *= rq; q1 *= rq;
      k0 *= rk; k1 *= rk;
      const float kq = wave_sum(q0 * k0 + q1 * k1);
      const float x0 = eA * (bf16_lo(gp) + dtb0);
      const float x1 = eA * (bf16_hi(gp) + dtb1);
      s_q[tt][2 * lane] = q0;
      s_q[tt][2 * lane + 1] = q1;
      s_k[tt][2 * lane] = k0;
      s_k[tt][2 * lane + 1] = k1;
      s_a[tt][2 * lane] = expf(p.lower_bound / (1.f + expf(-x0)));
      s_a[tt][2 * lane + 1] = expf(p.lower_bound / (1.f + expf(-x1)));
      if (lane < VS / 2) {
        reinterpret_cast<uint32_t*>(&s_v[tt][0])[lane] =
            reinterpret_cast<const uint32_t*>(p.v + t * p.ts_v + size_t(h) * p.hs_v + slice * VS)[lane];
      }
      if (lane == 0) {
        s_beta[tt] = 1.f / (1.f + expf(-bf16_to_f32(p.beta[t * p.ts_b + size_t(h) * p.hs_b])));
        s_kq[tt] = kq;
      }
    }
    __syncthreads();

    for (int tt = 0; tt < nt; ++tt) {
      // column sums over the 128 key rows in one fixed order for every split:
      // 16 groups of 8 rows (a sequential FMA chain each), then a pairwise tree
      // over the group index, low bits first -- the low levels in-lane, the
      // rest across the lanes of the column (xor shuffles; a+b == b+a exactly)
      float gk[GL], gq[GL];
#pragma unroll
      for (int gi = 0; gi < GL; ++gi) {
        float ak = 0.f, aq = 0.f;
#pragma unroll
        for (int i = gi * 8; i < gi * 8 + 8; i += 4) {
          const float4 a4 = *reinterpret_cast<const float4*>(&s_a[tt][r0 + i]);
          const float4 k4 = *reinterpret_cast<const float4*>(&s_k[tt][r0 + i]);
          const float4 q4 = *reinterpret_cast<const float4*>(&s_q[tt][r0 + i]);
          S[i] *= a4.x; S[i + 1] *= a4.y; S[i + 2] *= a4.z; S[i + 3] *= a4.w;
          ak = fmaf(S[i], k4.x, ak); ak = fmaf(S[i + 1], k4.y, ak);
          ak = fmaf(S[i + 2], k4.z, ak); ak = fmaf(S[i + 3], k4.w, ak);
          aq = fmaf(S[i], q4.x, aq); aq = fmaf(S[i + 1], q4.y, aq);
          aq = fmaf(S[i + 2], q4.z, aq); aq = fmaf(S[i + 3], q4.w, aq);
        }
        gk[gi] = ak;
        gq[gi] = aq;
      }
#pragma unroll
      for (int w = 1; w < GL; w *= 2)
#pragma unroll
        for (int gi = 0; gi < GL; gi += 2 * w) {
          gk[gi] += gk[gi + w];
          gq[gi] += gq[gi + w];
        }
      float pk = gk[0], pq = gq[0];
#pragma unroll
      for (int m = CW; m < 64; m <<= 1) {
        pk += __shfl_xor(pk, m, 64);
        pq += __shfl_xor(pq, m, 64);
      }
      const float d = s_beta[tt] * (bf16_to_f32(s_v[tt][jl]) - pk);
#pragma unroll
      for (int i = 0; i < R; i += 4) {
        const float4 k4 = *reinterpret_cast<const float4*>(&s_k[tt][r0 + i]);
        S[i] = fmaf(k4.x, d, S[i]); S[i + 1] = fmaf(k4.y, d, S[i + 1]);
        S[i + 2] = fmaf(k4.z, d, S[i + 2]); S[i + 3] = fmaf(k4.w, d, S[i + 3]);
      }
      if (rg == 0)
        p.out[size_t(t0 + tt) * p.ts_o + size_t(h) * p.hs_o + j] = f32_to_bf16(fmaf(s_kq[tt], d, pq));
      if (p.sp_idx) store_step(t0 + tt - bos);
    }
    __syncthreads();
  }

  if (p.sp_idx) return;  // a speculative-decode step stores per token only
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const size_t idx = sbase + (size_t)(r0 + i) * kD + j;
    if (p.state_bf16) static_cast<uint16_t*>(p.sT)[idx] = f32_to_bf16(S[i]);
    else static_cast<float*>(p.sT)[idx] = S[i];
  }
}

// The same recurrence for decode-sized calls, with 16-byte state accesses:
// wave w owns value columns [w CW, (w + 1) CW) of the slice (CW = VS / 4) and
// lane l owns the four columns 4 (l % C4) .. + 3 (C4 = CW / 4 quads) of the R
// consecutive key rows of row group l / C4.  The per-column arithmetic, and the
// order of every sum, are those of recurrent_kernel (8-row sequential groups,
// then a pairwise tree over the 16 group indices, low bits first), so both
// kernels give the same bits.  Tokens are staged 4 at a time.
template <int VS>
__global__ __launch_bounds__(kThreads) void decode_kernel(Params p) {
  constexpr int kTB = 4;
  constexpr int CW = VS / 4;    // value columns per wave
  constexpr int C4 = CW / 4;    // column quads per wave
  constexpr int RG = 64 / C4;   // row groups
  constexpr int R = kD / RG;    // key rows per lane
  constexpr int GL = R / 8;     // 8-row reduction groups per lane
  static_assert(R % 8 == 0, "rows per lane must be a multiple of 8");

  __shared__ float s_q[kTB][kD];
  __shared__ float s_k[kTB][kD];
  __shared__ float s_a[kTB][kD];
  __shared__ uint16_t s_v[kTB][VS];
  __shared__ float s_beta[kTB];
  __shared__ float s_kq[kTB];

  const int slice = blockIdx.x % p.vsplit;
  const int rest = blockIdx.x / p.vsplit;
  const int h = rest % p.H;
  const int n = p.order ? p.order[rest / p.H] : rest / p.H;
  const int H = p.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c4 = lane % C4, rg = lane / C4;
  const int jl = wave * CW + 4 * c4;  // first of this lane's columns inside the slice
  const int j = slice * VS + jl;      // ... as a value channel
  const int r0 = rg * R;              // first key row

  float4 S[R];
  const int64_t s0slot = start_slot(p, n);
  const size_t sbase = ((size_t)n * H + h) * kD * kD;
  const size_t s0base = ((size_t)max(s0slot, int64_t(0)) * H + h) * kD * kD;
  // the state after token i of a speculative-decode step, into its slot
  auto store_rows = [&](size_t b) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const size_t idx = b + (size_t)(r0 + i) * kD + j;
      if (p.state_bf16) {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.sT) + idx) =
            uint2{pack_bf16x2(S[i].x, S[i].y), pack_bf16x2(S[i].z, S[i].w)};
      } else {
        *reinterpret_cast<float4*>(static_cast<float*>(p.sT) + idx) = S[i];
      }
    }
  };
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const size_t idx = s0base + (size_t)(r0 + i) * kD + j;
    if (!p.s0 || s0slot < 0) {
      S[i] = float4{0.f, 0.f, 0.f, 0.f};
    } else if (p.state_bf16) {
      const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p.s0) + idx);
      S[i] = float4{bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
    } else {
      S[i] = *reinterpret_cast<const float4*>(static_cast<const float*>(p.s0) + idx);
    }
  }

  const float eA = expf(p.A_log[h]);
  const float dtb0 = p.dt_bias[h * kD + 2 * lane];
  const float dtb1 = p.dt_bias[h * kD + 2 * lane + 1];
  // the bounds are uniform: scalar registers (else every buffer access with a
  // token offset in its scalar operand becomes a loop over lanes)
  const int bos = __builtin_amdgcn_readfirstlane(min(max(p.cu[n], 0), p.T));
  const int eos = __builtin_amdgcn_readfirstlane(min(max(p.cu[n + 1], bos), p.T));

  for (int t0 = bos; t0 < eos; t0 += kTB) {
    const int nt = min(kTB, eos - t0);
    for (int tt = wave; tt < nt; tt += 4) {
      const size_t t = size_t(t0 + tt);
      const uint32_t qp = reinterpret_cast<const uint32_t*>(p.q + t * p.ts_q + size_t(h) * p.hs_q)[lane];
      const uint32_t kp = reinterpret_cast<const uint32_t*>(p.k + t * p.ts_k + size_t(h) * p.hs_k)[lane];
      const uint32_t gp = reinterpret_cast<const uint32_t*>(p.g + t * p.ts_g + size_t(h) * p.hs_g)[lane];
      float q0 = bf16_lo(qp), q1 = bf16_hi(qp);
      float k0 = bf16_lo(kp), k1 = bf16_hi(kp);
      const float rq = rsqrtf(wave_sum(q0 * q0 + q1 * q1) + kNormEps) * p.scale;
      const float rk = rsqrtf(wave_sum(k0 * k0 + k1 * k1) + kNormEps);
      q0 *= rq; q1 *= rq;
      k0 *= rk; k1 *= rk;
      const float kq = wave_sum(q0 * k0 + q1 * k1);
      const float x0 = eA * (bf16_lo(gp) + dtb0);
      const float x1 = eA * (bf16_hi(gp) + dtb1);
      s_q[tt][2 * lane] = q0;
      s_q[tt][2 * lane + 1] = q1;
      s_k[tt][2 * lane] = k0;
      s_k[tt][2 * lane + 1] = k1;
      s_a[tt][2 * lane] = expf(p.lower_bound / (1.f + expf(-x0)));
      s_a[tt][2 * lane + 1] = expf(p.lower_bound / (1.f + expf(-x1)));
      if (lane < VS / 2) {
        reinterpret_cast<uint32_t*>(&s_v[tt][0])[lane] =
            reinterpret_cast<const uint32_t*>(p.v + t * p.ts_v + size_t(h) * p.hs_v + slice * VS)[lane];
      }
      if (lane == 0) {
        s_beta[tt] = 1.f / (1.f + expf(-bf16_to_f32(p.beta[t * p.ts_b + size_t(h) * p.hs_b])));
        s_kq[tt] = kq;
      }
    }
    __syncthreads();

    for (int tt = 0; tt < nt; ++tt) {
      float4 gk[GL], gq[GL];
#pragma unroll
      for (int gi = 0; gi < GL; ++gi) {
        float4 ak = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = gi * 8; i < gi * 8 + 8; ++i) {
          const float a = s_a[tt][r0 + i], kk = s_k[tt][r0 + i], qq = s_q[tt][r0 + i];
          S[i].x *= a; S[i].y *= a; S[i].z *= a; S[i].w *= a;
          ak.x = fmaf(S[i].x, kk, ak.x); ak.y = fmaf(S[i].y, kk, ak.y);
          ak.z = fmaf(S[i].z, kk, ak.z); ak.w = fmaf(S[i].w, kk, ak.w);
          aq.x = fmaf(S[i].x, qq, aq.x); aq.y = fmaf(S[i].y, qq, aq.y);
          aq.z = fmaf(S[i].z, qq, aq.z); aq.w = fmaf(S[i].w, qq, aq.w);
        }
        gk[gi] = ak;
        gq[gi] = aq;
      }
#pragma unroll
      for (int w = 1; w < GL; w *= 2)
#pragma unroll
        for (int gi = 0; gi < GL; gi += 2 * w) {
          gk[gi].x += gk[gi + w].x; gk[gi].y += gk[gi + w].y;
          gk[gi].z += gk[gi + w].z; gk[gi].w += gk[gi + w].w;
          gq[gi].x += gq[gi + w].x; gq[gi].y += gq[gi + w].y;
          gq[gi].z += gq[gi + w].z; gq[gi].w += gq[gi + w].w;
        }
      float4 pk = gk[0], pq = gq[0];
#pragma unroll
      for (int m = C4; m < 64; m <<= 1) {
        pk.x += __shfl_xor(pk.x, m, 64); pk.y += __shfl_xor(pk.y, m, 64);
        pk.z += __shfl_xor(pk.z, m, 64); pk.w += __shfl_xor(pk.w, m, 64);
        pq.x += __shfl_xor(pq.x, m, 64); pq.y += __shfl_xor(pq.y, m, 64);
        pq.z += __shfl_xor(pq.z, m, 64); pq.w += __shfl_xor(pq.w, m, 64);
      }
      const float b = s_beta[tt];
      const float4 d = {b * (bf16_to_f32(s_v[tt][jl]) - pk.x), b * (bf16_to_f32(s_v[tt][jl + 1]) - pk.y),
                        b * (bf16_to_f32(s_v[tt][jl + 2]) - pk.z), b * (bf16_to_f32(s_v[tt][jl + 3]) - pk.w)};
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const float kk = s_k[tt][r0 + i];
        S[i].x = fmaf(kk, d.x, S[i].x); S[i].y = fmaf(kk, d.y, S[i].y);
        S[i].z = fmaf(kk, d.z, S[i].z); S[i].w = fmaf(kk, d.w, S[i].w);
      }
      if (rg == 0) {
        const float kq = s_kq[tt];
        const uint2 o = {pack_bf16x2(fmaf(kq, d.x, pq.x), fmaf(kq, d.y, pq.y)),
                         pack_bf16x2(fmaf(kq, d.z, pq.z), fmaf(kq, d.w, pq.w))};
        *reinterpret_cast<uint2*>(p.out + size_t(t0 + tt) * p.ts_o + size_t(h) * p.hs_o + j) = o;
      }
      if (p.sp_idx) {
        const int64_t slot = step_slot(p, n, t0 + tt - bos);
        if (slot >= 0) store_rows(((size_t)slot * H + h) * kD * kD);
      }
    }
    __syncthreads();
  }

  if (!p.sp_idx) store_rows(sbase);  // a speculative-decode step stores per token only
}

}  // namespace

hipError_t launch_recurrent(const Params& p, hipStream_t stream, bool decode) {
  const void* fn = nullptr;
  switch (kD / p.vsplit) {
    // decode staging: 16-byte state accesses where a wave's columns hold
    // whole 8-row groups per lane (slices of 64 or 128 columns)
    case 128:
      fn = decode ? reinterpret_cast<const void*>(&decode_kernel<128>)
                  : reinterpret_cast<const void*>(&recurrent_kernel<128, 32>);
      break;
    case 64:
      fn = decode ? reinterpret_cast<const void*>(&decode_kernel<64>)
                  : reinterpret_cast<const void*>(&recurrent_kernel<64, 32>);
      break;
    case 32:
      fn = decode ? reinterpret_cast<const void*>(&recurrent_kernel<32, 4>)
                  : reinterpret_cast<const void*>(&recurrent_kernel<32, 32>);
      break;
    case 16:
      fn = decode ? reinterpret_cast<const void*>(&recurrent_kernel<16, 4>)
                  : reinterpret_cast<const void*>(&recurrent_kernel<16, 32>);
      break;
    default: return hipErrorInvalidValue;
  }
  Params arg = p;
  void* args[] = {&arg};
  // the launch status comes from this call alone, not from an earlier runtime call
  return hipLaunchKernel(fn, dim3(p.N * p.H * p.vsplit), dim3(kThreads), args, 0, stream);
}

}  // namespace kda
