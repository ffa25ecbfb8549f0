// kda_duo.hip -- the pipelined 16-token forward with its two roles in two
// workgroups of one XCD: for each (sequence, head) item, a producer workgroup
// builds every chunk's package once and a consumer workgroup walks the state
// over all 128 value columns.
//
// The single-workgroup kernel (kda_pipe.hip) holds at most 64 value columns
// of state per workgroup, so with 128 columns each item takes two workgroups
// and both repeat all of the item's state-independent work (norms, gate,
// decays, the inverse, M'), which is most of the kernel's instruction issue.
// Here the two CUs of an item do different work: the producer CU forms each
// package once and hands it to the consumer CU through the XCD's L2.
//
// Pairing.  Workgroup B = 16 (i / 8) + 8 role + i % 8 for item i: the two
// workgroups of an item are 8 indices apart, so they run on one XCD
// (workgroup B runs on XCD (B + o) mod 8 for an offset o shared by the grid)
// and meet in its L2.  The launch is taken only when the whole grid fits on
// the device at once (one workgroup per CU by its LDS size, 2 N H <= CUs).
// An XCD starts its workgroups in index order, producer, consumer, producer,
// consumer, ..., so a consumer never waits for a producer that has not been
// started.
//
// Producer workgroup: ten producer waves build the packages of five chunk
// slots in LDS, two waves a chunk (the 64-channel halves, as in the
// single-workgroup kernel); two copy waves (even and odd chunks) copy each
// finished package into the item's ring of kDuoRing (4) packages in the
// workspace, slot chunk mod kDuoRing, once the consumer has taken the package
// that last held it, wait for their stores, and publish the count of their
// chunks in a flag word.  A short ring keeps each slot's reuse within what
// the XCD's L2 holds: with 8 slots most packages were written back to HBM
// before they were read.
//
// Consumer workgroup: eight state waves (one 16-column strip each) and two
// loader waves (even and odd chunks, matching the copy waves).  A loader
// copies each published package of its parity from the ring into an LDS ring
// of eight slots (two buffers of four, which the state waves walk as the
// single-workgroup kernel walks its package buffers) with loads straight into
// LDS, waits for them, counts the package in the slot's LDS counter and
// acknowledges it in its flag word (the ring slot may be refilled).  A loader
// reads LDS (the slot counters) only while none of its loads is in flight:
// the compiler waits for every load into LDS before any LDS access of the
// wave, so a second package in flight has to be the other loader's.
//
// Flags: one uint64 word per writer, (nonce << 32) | (xcc << 28) | count.
// The nonce is a per-call value from the host, so words left by an earlier
// call (or other data of the workspace) are never taken for this call's; each
// loader clears its parity's two words when it is done, so a graph replayed
// with the same nonce starts from zero again.  xcc is the XCD of the publishing
// workgroup: the loader checks it against its own (a pair split over two XCDs
// would not see each other's stores in one L2) and reports a mismatch in the
// status word (2).  Polls read the words with scalar loads that bypass the
// scalar cache (glc): they count on their own counter, so a poll never waits
// for the wave's package loads or stores.  Every wait is bounded like the
// LDS waits: giving up marks the workgroup's LDS error word, every later wait
// returns at once and the status word is set (1).
#include "kda_pipe_parts.h"

namespace kda {
namespace {

constexpr int kDuoSlots = 5;                    // chunk slots of the producer workgroup
constexpr int kDuoProd = kDuoSlots * kPH;       // producer waves
constexpr int kDuoCopy = 2;                     // copy waves (even, odd chunks)
constexpr int kDuoLoaders = kDuoCopy;           // loader waves (even, odd chunks)
constexpr int kDuoStrips = 8;                   // state waves (16 value columns each)
constexpr int kDuoRound = 4;                    // chunks per LDS buffer of the consumer
constexpr int kDuoThreads = 64 * (kDuoProd + kDuoCopy);
constexpr int kPkgWords = sizeof(Pack) / 16;    // 16-byte words of a package
constexpr int kPkgLoads = (kPkgWords + 63) / 64;  // 1 KB blocks (one 16-byte load per lane each)
static_assert(kDuoStrips + kDuoLoaders <= kDuoProd + kDuoCopy, "the consumer's waves fit the block");
static_assert(kDuoRing % kDuoCopy == 0, "a ring slot holds chunks of one parity");
static_assert(kDuoRing % kDuoCopy == 0, "a ring slot holds chunks of one parity");
static_assert(kPkgLoads * 1024 == kDuoPkgBytes, "ring slots hold whole 1 KB blocks");

// A package in the consumer's LDS ring, padded to whole 1 KB blocks.
struct LPack {
  Pack p;
  unsigned char pad[kDuoPkgBytes - sizeof(Pack)];
};

struct ProdSmem {
  Pack pk[kDuoSlots];
  bf16 kg[kDuoSlots][128 * kTok];  // K_G, swizzled rows
  int half[kDuoSlots];             // producer-half syncs (both halves, once a round)
  int rdy[kDuoSlots];              // finished package parts (both halves, once a round)
  int copied[kDuoSlots];           // packages copied out of the slot
  int err;
};

struct ConsSmem {
  LPack pk[2][kDuoRound];   // first: keeps the packages' alignment
  Tiles t[kDuoStrips];
};

// The consumer's LDS counters, in an LDS object of their own: the loader's
// counter accesses then provably miss the packages its loads write into LDS,
// so the compiler does not wait for those loads before each of them.
struct ConsSync {
  int done[kDuoRound][kDuoStrips];  // per slot: rounds each state wave is done with
  int lrdy[2][kDuoRound];           // per slot: packages loaded into it
  int err;
};

union DuoSmem {
  ProdSmem p;
  ConsSmem c;
};

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt at their maximum: no wait), as the
// builtin, so the compiler knows the wave's loads into LDS are complete.
constexpr int kVmcnt0 = 0x0F70;

__device__ __forceinline__ uint64_t flag_word(uint32_t nonce, int xcc, int count) {
  return (uint64_t(nonce) << 32) | (uint64_t(xcc & 15) << 28) | uint64_t(uint32_t(count) & 0x0fffffffu);
}

// The word at p, through a scalar load that bypasses the scalar cache (glc);
// the wait is in the same asm block, so the result registers are never
// live while the load is in flight.
__device__ __forceinline__ uint64_t poll_word(const uint64_t* p) {
  uint64_t v;
  asm volatile("s_load_dwordx2 %0, %1, 0x0 glc\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  return v;
}

// Wait until the flag word at f carries this call's nonce and a count of at
// least target; returns the count seen (0 after giving up).  *xcc_seen gets
// the publisher's XCD.
__device__ __forceinline__ int wait_flag(const uint64_t* f, uint32_t nonce, int target, int* err,
                                         int* xcc_seen) {
  if (gave_up(err)) return 0;
#pragma unroll 1
  for (int it = 0; it < kSpinMax; ++it) {
    const uint64_t w = poll_word(f);
    const int cnt = int(uint32_t(w) & 0x0fffffffu);
    if (uint32_t(w >> 32) == nonce && cnt >= target) {
      *xcc_seen = int((uint32_t(w) >> 28) & 15u);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      return cnt;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  return 0;
}

// Flag stores from lane 0, through L2 (agent scope: sc1), as global (not
// flat) stores, so they count on the vector memory counter only.
__device__ __forceinline__ void store_flag(uint64_t* f, uint64_t w, int lane) {
  typedef __attribute__((address_space(1))) uint64_t gword;
  if (lane == 0) __hip_atomic_store((gword*)f, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// A pointer that is the same in every lane, in scalar registers (the scalar
// polls take their address from there).
// (readfirstlane returns a signed int: each half goes through uint32_t, or
// a low half with bit 31 set would be sign-extended into the high one.)
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* q) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(q);
  const uint32_t lo = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(a))));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(a >> 32))));
  return reinterpret_cast<T*>(uint64_t(lo) | (uint64_t(hi) << 32));
}

// Status word: 1 a bounded wait gave up, 2 a pair on two XCDs (the larger
// kind stays).
__device__ __forceinline__ void report(int32_t* errword, int kind) {
  __hip_atomic_fetch_max(errword, kind, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int xcc_id() {
  int x;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
  return x & 15;
}

__global__ __launch_bounds__(kDuoThreads, 1) void duo_kernel(Params p) {
  __shared__ __attribute__((aligned(16))) DuoSmem sm;
  __shared__ __attribute__((aligned(16))) ConsSync csy;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;

  const int B = blockIdx.x;
  const int role = (B >> 3) & 1;  // 0 producer, 1 consumer
  const int item = 8 * (B >> 4) + (B & 7);
  const int H = p.H;
  if (item >= p.N * H) return;  // the whole workgroup
  const int n = item / H, h = item % H;
  const int bos = __builtin_amdgcn_readfirstlane(min(max(p.cu[n], 0), p.T));
  const int eos = __builtin_amdgcn_readfirstlane(min(max(p.cu[n + 1], bos), p.T));
  const int nc = (eos - bos + kTok - 1) / kTok;
  const int xcc = xcc_id();

  // the item's flag words: published counts of the even and the odd chunks
  // (the copy waves), loaded counts of the even and the odd chunks (the loaders)
  uint64_t* flags = uniform_ptr(p.duo_flags + kDuoFlagWords * size_t(item));
  const __amdgpu_buffer_rsrc_t ring = __builtin_amdgcn_make_buffer_rsrc(
      static_cast<char*>(p.duo_ring) + size_t(item) * kDuoRing * kDuoPkgBytes, (short)0,
      kDuoRing * kDuoPkgBytes, kRsrcWord3);

  // LDS counters to zero (both roles), before any wave leaves
  {
    int* ctr = role == 0 ? &sm.p.half[0] : &csy.done[0][0];
    const int nctr = role == 0 ? 3 * kDuoSlots + 1 : kDuoRound * kDuoStrips + 2 * kDuoRound + 1;
    if (tid < nctr) ctr[tid] = 0;
  }
  __syncthreads();

  if (role == 0) {
    // ---------------- producer workgroup ----------------
    ProdSmem& sp = sm.p;
    const int nr = (nc + kDuoSlots - 1) / kDuoSlots;
    auto producer = [&](auto half) {
      constexpr int hf = decltype(half)::value;
      const int c = wave - kDuoSlots * hf;
      RawSrc src;
      src.q = rows_rsrc(p.q + size_t(h) * p.hs_q, eos, p.ts_q, kD);
      src.k = rows_rsrc(p.k + size_t(h) * p.hs_k, eos, p.ts_k, kD);
      src.g = rows_rsrc(p.g + size_t(h) * p.hs_g, eos, p.ts_g, kD);
      src.qn = rows_rsrc(p.q + size_t(h) * p.hs_q, hf ? eos : 0, p.ts_q, kD);
      src.beta = rows_rsrc(p.beta + size_t(h) * p.hs_b, hf ? 0 : eos, p.ts_b, 1);
      const float eA = expf(p.A_log[h]);
      const float c1 = -kLog2e * eA;
      const float lb2 = p.lower_bound * kLog2e;
      float c2[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) c2[i] = c1 * p.dt_bias[h * kD + 64 * hf + 4 * (lane & 15) + i];
      __builtin_amdgcn_sched_barrier(0);
      const RawLoad ld{src, p.ts_q, p.ts_k, p.ts_g, p.ts_b, lane, hf};
      Raw raw;
      ld.all(raw, bos + kTok * c);
      for (int r = 0; r < nr; ++r) {
        const int j = kDuoSlots * r + c;
        if (j >= nc) break;
        Pack& P = sp.pk[c];
        bf16* kg = sp.kg[c];
        // the slot is free once its previous package has been copied out
        // (the copy waited for both halves' second phase, the last reads of kg)
        if (r >= 1) wait_count(&sp.copied[c], r, &sp.err);
        const int t0 = bos + kTok * j, Lc = min(kTok, eos - t0);
        const int tn = t0 + kTok * kDuoSlots;
        produce_operands<false, false>(P, kg, raw, ld, tn, hf, Lc, lane, c2, c1, lb2, p.scale);
        arrive(&sp.half[c], lane);
        wait_count(&sp.half[c], kPH * (r + 1), &sp.err);
        if (hf == 0) produce_inverse(P, kg, lane);
        else produce_m(P, kg, lane);
        arrive(&sp.rdy[c], lane);
      }
    };
    if (wave < kDuoSlots) {
      producer(BufIdx<0>{});
    } else if (wave < kDuoProd) {
      producer(BufIdx<1>{});
    } else {
      // copy wave cw: chunks cw, cw + 2, ...
      __builtin_amdgcn_s_setprio(1);
      const int cw = wave - kDuoProd;
      const uint64_t* ackp = flags + 2 + cw;  // its chunks' loader
      int acked = 0, xs = 0;
      for (int j = cw; j < nc; j += kDuoCopy) {
        const int c = j % kDuoSlots, r = j / kDuoSlots;
        wait_count(&sp.rdy[c], kPH * (r + 1), &sp.err);
        // ring slot j % kDuoRing is free once the consumer took chunk j -
        // kDuoRing (the same parity: its loader counts it)
        if (j >= kDuoRing && acked < (j - kDuoRing) / kDuoCopy + 1)
          acked = wait_flag(ackp, p.duo_nonce, (j - kDuoRing) / kDuoCopy + 1, &sp.err, &xs);
        uint4 d[kPkgLoads];
        const uint4* src = reinterpret_cast<const uint4*>(&sp.pk[c]);
#pragma unroll
        for (int i = 0; i < kPkgLoads; ++i) {
          const int w = 64 * i + lane;
          d[i] = w < kPkgWords ? src[w] : uint4{0u, 0u, 0u, 0u};
        }
        arrive(&sp.copied[c], lane);  // (its release waits for the LDS reads)
        const unsigned base = unsigned(j % kDuoRing) * unsigned(kDuoPkgBytes);
#pragma unroll
        for (int i = 0; i < kPkgLoads; ++i)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, d[i]), ring,
                                                 base + 1024u * i + 16u * lane, 0, 0);
        // the package is in L2 before its count is
        __builtin_amdgcn_s_waitcnt(kVmcnt0);
        store_flag(flags + cw, flag_word(p.duo_nonce, xcc, j / kDuoCopy + 1), lane);
      }
    }
    if (lane == 0 && gave_up(&sp.err)) report(p.errword, 1);
    return;
  }

  // ---------------- consumer workgroup ----------------
  ConsSmem& cs = sm.c;
  const int nr = (nc + kDuoRound - 1) / kDuoRound;
  if (wave >= kDuoStrips + kDuoLoaders) return;
  if (wave >= kDuoStrips) {
    // loader lw: chunks j = lw, lw + 2, ... (the chunks copy wave lw
    // publishes), each into LDS slot (j / 4 % 2, j % 4); the two loaders keep
    // two packages in flight
    __builtin_amdgcn_s_setprio(1);
    const int lw = wave - kDuoStrips;
    int known = 0;  // published count seen
    for (int j = lw; j < nc; j += kDuoLoaders) {
      const int r = j / kDuoRound, c = j % kDuoRound;
      // every state wave is done with the slot's previous package (round r - 2)
      if (r >= 2) {
        wait_row<4>(&csy.done[c][0], r - 1, &csy.err);
        wait_row<4>(&csy.done[c][4], r - 1, &csy.err);
      }
      // chunk j is in the ring
      const int need = j / kDuoCopy + 1;
      if (known < need) {
        int xs = xcc;
        known = wait_flag(flags + lw, p.duo_nonce, need, &csy.err, &xs);
        if (xs != xcc) {
          __hip_atomic_store(&csy.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          if (lane == 0) report(p.errword, 2);
        }
      }
      // from the ring (through L2: sc1) straight into the LDS slot, 1 KB a load
      char* dst = reinterpret_cast<char*>(&cs.pk[r & 1][c]);
      const unsigned base = unsigned(j % kDuoRing) * unsigned(kDuoPkgBytes);
#pragma unroll
      for (int i = 0; i < kPkgLoads; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ring, (__attribute__((address_space(3))) void*)(dst + 1024 * i), 16, 16u * unsigned(lane),
            base + 1024u * i, 0, 16 /* sc1 */);
      __builtin_amdgcn_s_waitcnt(kVmcnt0);
      arrive(&csy.lrdy[r & 1][c], lane);
      // the ring slot may be refilled
      store_flag(flags + 2 + lw, flag_word(p.duo_nonce, xcc, j / kDuoLoaders + 1), lane);
    }
    // every package of this parity is taken (so its copy wave stores and
    // polls nothing more): clear the two words for the next call
    store_flag(flags + lw, 0, lane);
    store_flag(flags + 2 + lw, 0, lane);
    if (lane == 0 && gave_up(&csy.err)) report(p.errword, 1);
    return;
  }

  // state waves: strip sw, value columns 16 sw .. 16 sw + 15
  const int sw = wave;
  const int colb = 16 * sw + l16;
  const __amdgpu_buffer_rsrc_t vsrc = rows_rsrc(p.v + size_t(h) * p.hs_v, eos, p.ts_v, kD);
  const __amdgpu_buffer_rsrc_t odst = rows_rsrc(p.out + size_t(h) * p.hs_o, eos, p.ts_o, kD);
  const size_t sbase = (size_t(n) * H + h) * kD * kD;
  f32x4 S[8];
  if (!p.s0) {
#pragma unroll
    for (int rt = 0; rt < 8; ++rt) S[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  } else if (p.state_bf16) {
    const uint16_t* s0 = static_cast<const uint16_t*>(p.s0) + sbase + colb;
    uint16_t raw0[8][4];
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int j = 0; j < 4; ++j) raw0[rt][j] = s0[(16 * rt + 4 * g4 + j) * kD];
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int j = 0; j < 4; ++j) S[rt][j] = bf16_to_f32(raw0[rt][j]);
  } else {
    const float* s0 = static_cast<const float*>(p.s0) + sbase + colb;
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int j = 0; j < 4; ++j) S[rt][j] = s0[(16 * rt + 4 * g4 + j) * kD];
  }
  const unsigned cstrip = unsigned(16 * sw);
  uint2 va[kDuoRound], vbuf[kDuoRound];
#pragma unroll
  for (int c = 0; c < kDuoRound; ++c) va[c] = vbuf[c] = uint2{0u, 0u};
  auto load_round = [&](uint2 (&v)[kDuoRound], int r) {
#pragma unroll
    for (int c = 0; c < kDuoRound; ++c) v[c] = load_vrow(vsrc, cstrip, p.ts_v, bos + kTok * (kDuoRound * r + c), lane);
  };
  Tiles& tl = cs.t[sw];
  auto consume_round = [&](const uint2 (&v)[kDuoRound], int r, auto buf) {
    constexpr int Bf = decltype(buf)::value;
#pragma unroll
    for (int c = 0; c < kDuoRound; ++c) {
      const int j = kDuoRound * r + c;
      if (j >= nc) break;
      wait_count(&csy.lrdy[Bf][c], (r >> 1) + 1, &csy.err);
      const Pack& P = cs.pk[Bf][c].p;
      const int t0 = bos + kTok * j;
      bf16x8 ax[4], aq[4];
#pragma unroll
      for (int kb2 = 0; kb2 < 4; ++kb2) {
        const int r1 = 32 * kb2 + 4 * g4 + (l16 >> 2), r2 = r1 + 16;
        const int o1 = tile(r1, l16 & 3), o2 = tile(r2, l16 & 3);
        ax[kb2] = cat(tr4(&P.x[o1]), tr4(&P.x[o2]));
        aq[kb2] = cat(tr4(&P.qt[o1]), tr4(&P.qt[o2]));
      }
      const f32x4 bR = *reinterpret_cast<const f32x4*>(&P.beta[4 * g4]);
      const f32x4 rqR = *reinterpret_cast<const f32x4*>(&P.rqs[4 * g4]);
      const bf16x4 Lf = *reinterpret_cast<const bf16x4*>(&P.l[frag(0, l16, 4 * g4)]);
      const bf16x4 Mf = *reinterpret_cast<const bf16x4*>(&P.m[frag(0, l16, 4 * g4)]);
      *reinterpret_cast<uint2*>(&tl.v[4 * lane]) = v[c];
      __builtin_amdgcn_wave_barrier();
      const f32x4 V = to_f32x4(tr4(&tl.v[4 * lane]));

      bf16x8 Sb[4];
#pragma unroll
      for (int kb2 = 0; kb2 < 4; ++kb2) Sb[kb2] = cat(to_bf16x4(S[2 * kb2]), to_bf16x4(S[2 * kb2 + 1]));
      f32x4 Y = {0.f, 0.f, 0.f, 0.f}, Q = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb2 = 0; kb2 < 4; ++kb2) {
        Y = mfma32(ax[kb2], Sb[kb2], Y);
        Q = mfma32(aq[kb2], Sb[kb2], Q);
      }
      asm volatile("" : "+v"(Y), "+v"(Q));
      {
        const float2 gv = *reinterpret_cast<const float2*>(&P.gam[16 * (l16 >> 1) + 4 * g4 + 2 * (l16 & 1)]);
        decay_strip(S, gv.x, gv.y);
      }
      asm volatile("" : "+v"(S[0]), "+v"(S[1]), "+v"(S[2]), "+v"(S[3]), "+v"(S[4]), "+v"(S[5]),
                   "+v"(S[6]), "+v"(S[7]), "+v"(Y), "+v"(Q));
      const f32x4 D = V - Y;
      const f32x4 N = mfma16(Lf, to_bf16x4(D), bR * D);
      const f32x4 O = mfma16(Mf, to_bf16x4(N), rqR * Q);
      *reinterpret_cast<uint2*>(&tl.o[16 * l16 + 4 * g4]) = uint2{pk2(O[0], O[1]), pk2(O[2], O[3])};
      __builtin_amdgcn_wave_barrier();
      const bf16x4 orow = tr4(&tl.o[64 * g4 + 16 * (l16 >> 2) + 4 * (l16 & 3)]);
      __builtin_amdgcn_raw_buffer_store_b64(
          __builtin_bit_cast(u32x2, orow), odst,
          ((unsigned(t0) + unsigned(l16)) * unsigned(p.ts_o) + cstrip + 4u * g4) * 2u, 0, 0);
      const f16x4 Nq = f16x4{(_Float16)(N[0] * kNScale), (_Float16)(N[1] * kNScale),
                             (_Float16)(N[2] * kNScale), (_Float16)(N[3] * kNScale)};
#pragma unroll
      for (int rt = 0; rt < 8; ++rt) {
        const f16x4 a = *reinterpret_cast<const f16x4*>(&P.kp[fragx(rt, l16, 4 * g4)]);
        S[rt] = mfma16h(a, Nq, S[rt]);
      }
      arrive(&csy.done[c][sw], lane);
    }
  };

  load_round(va, 0);
  for (int r = 0; r < nr; r += 2) {
    load_round(vbuf, r + 1);
    consume_round(va, r, BufIdx<0>{});
    if (r + 1 < nr) {
      load_round(va, r + 2);
      consume_round(vbuf, r + 1, BufIdx<1>{});
    }
  }
  // final state (in the state dtype)
  if (p.state_bf16) {
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        static_cast<bf16*>(p.sT)[sbase + size_t(16 * rt + 4 * g4 + j) * kD + colb] = (bf16)S[rt][j];
  } else {
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        static_cast<float*>(p.sT)[sbase + size_t(16 * rt + 4 * g4 + j) * kD + colb] = S[rt][j];
  }
  if (lane == 0 && gave_up(&csy.err)) report(p.errword, 1);
}

}  // namespace

hipError_t launch_duo(const Params& p, hipStream_t stream) {
  const int items = (p.N * p.H + 7) / 8 * 8;
  Params arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&duo_kernel), dim3(2 * items), dim3(kDuoThreads),
                         args, 0, stream);
}

}  // namespace kda
