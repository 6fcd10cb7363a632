// mk_device.h -- device building blocks for gfx950 (CDNA4): the bf16 matrix-core
// tile GEMM, the peer-reduce of one region, tile readiness flags and timers.
//
// The tile GEMM follows the compute role of Figure 2 (item 1) on the
// thelatestinai.com page of "mKernel: Fast Multi-GPU, Multi-Node Fused Kernels":
// a workgroup computes one output tile and stores it to device memory. The
// reduce follows the communication role (items 2 and 6): once a tile is ready,
// add the other GPUs' partials of that tile. On one GPU the peers' partials are
// inputs already in HBM.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kThreads = 256;  // 4 waves of 64 lanes

// ----------------------------------------------------------------- conversions

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float -> bfloat16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// ----------------------------------------------------------------- timers, flags

// Constant 100 MHz clock shared by all compute units.
__device__ __forceinline__ uint64_t ticks() { return __builtin_amdgcn_s_memrealtime(); }

// Readiness flag protocol (Figure 2, item 1: "write completed tiles to GPU
// memory and set readiness flags"; Table 2's caption: completion of a transfer
// and visibility in GPU memory are separate requirements). Every thread of the
// producing workgroup has stored its part of the tile; the barrier orders those
// stores before thread 0's agent-scope release store of the flag, so a consumer
// on any XCD that acquires the flag sees the whole tile.
__device__ __forceinline__ void publish_flag(int* flag, int epoch) {
  __hip_atomic_store(flag, epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int load_relaxed(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void acquire_fence() {
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// ----------------------------------------------------------------- tile GEMM

// Tile shape: BM x BN outputs per workgroup, BK = 64 k-values per stage.
// Four waves in a 2 x 2 arrangement; each wave owns a (BM/2) x (BN/2) block made
// of 32 x 32 matrix-core blocks (v_mfma_f32_32x32x16_bf16).
// LDS layout, double-buffered:
//   As[BM][BK+8]   A tile, k contiguous (row pitch 144 B spreads 16 rows over all banks)
//   Bs[BK][BN+32]  B tile, n contiguous, read with the gfx950 transposing LDS load
template <int BM_, int BN_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = 64;
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int AP = BK + 8;
  static constexpr int BP = BN + 32;
  static constexpr int A_ELEMS = BM * AP;
  static constexpr int B_ELEMS = BK * BP;
  static constexpr int STAGE = A_ELEMS + B_ELEMS;  // bf16 elements per stage
  static constexpr int LDS_BYTES = 2 * STAGE * 2;
  static constexpr int A_LD = BM * BK / 8 / kThreads;  // 16-byte chunks per thread
  static constexpr int B_LD = BK * BN / 8 / kThreads;
  static_assert(FM >= 1 && FN >= 1, "tile too small");
  static_assert(A_LD >= 1 && B_LD >= 1, "tile too small for 256 threads");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// Tile index -> (tile row, tile column), grouped so that consecutive tiles share
// A row-panels (GROUP rows of tiles sweep the columns together).
__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int GROUP = 8;
  int group_size = GROUP * tiles_n;
  int g = t / group_size;
  int first = g * GROUP;
  int gm = tiles_m - first < GROUP ? tiles_m - first : GROUP;
  int w = t - g * group_size;
  tm = first + w % gm;
  tn = w / gm;
}

template <class Cfg>
struct GemmTile {
  f32x16 acc[Cfg::FM][Cfg::FN];
  u32x4 ra[Cfg::A_LD];
  u32x4 rb[Cfg::B_LD];

  __device__ __forceinline__ void load_global(const uint16_t* __restrict__ A,
                                              const uint16_t* __restrict__ B, int64_t M, int64_t N,
                                              int64_t K, int64_t m0, int64_t n0, int64_t k0,
                                              int tid) {
#pragma unroll
    for (int c = 0; c < Cfg::A_LD; ++c) {
      int idx = c * kThreads + tid;
      int row = idx >> 3;  // BK/8 = 8 chunks per row
      int kc = idx & 7;
      int64_t gm = m0 + row, gk = k0 + kc * 8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (gm < M && gk < K) v = *(const u32x4*)(A + gm * K + gk);
      ra[c] = v;
    }
    constexpr int CPR = Cfg::BN / 8;  // chunks per B row
#pragma unroll
    for (int c = 0; c < Cfg::B_LD; ++c) {
      int idx = c * kThreads + tid;
      int row = idx / CPR;
      int nc = idx % CPR;
      int64_t gk = k0 + row, gn = n0 + nc * 8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (gk < K && gn < N) v = *(const u32x4*)(B + gk * N + gn);
      rb[c] = v;
    }
  }

  __device__ __forceinline__ void store_lds(uint16_t* stage, int tid) {
    uint16_t* As = stage;
    uint16_t* Bs = stage + Cfg::A_ELEMS;
#pragma unroll
    for (int c = 0; c < Cfg::A_LD; ++c) {
      int idx = c * kThreads + tid;
      *(u32x4*)(As + (idx >> 3) * Cfg::AP + (idx & 7) * 8) = ra[c];
    }
    constexpr int CPR = Cfg::BN / 8;
#pragma unroll
    for (int c = 0; c < Cfg::B_LD; ++c) {
      int idx = c * kThreads + tid;
      *(u32x4*)(Bs + (idx / CPR) * Cfg::BP + (idx % CPR) * 8) = rb[c];
    }
  }

  // 4 steps of k=16 on one LDS stage.
  __device__ __forceinline__ void mma_stage(const uint16_t* stage, int wave, int lane) {
    const uint16_t* As = stage;
    const uint16_t* Bs = stage + Cfg::A_ELEMS;
    const int wm = wave >> 1, wn = wave & 1;
    const int arow = wm * Cfg::WM + (lane & 31);
    const int akof = (lane >> 5) * 8;
    // transposing read: 16-lane group g reads a 4(k) x 16(n) block per instruction;
    // lane r of the group supplies row r/4, columns 4*(r%4) .. +3.
    const int g = lane >> 4, r = lane & 15;
    const int bk = (g >> 1) * 8 + (r >> 2);
    const int bn = wn * Cfg::WN + (g & 1) * 16 + 4 * (r & 3);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 a[Cfg::FM], b[Cfg::FN];
#pragma unroll
      for (int fm = 0; fm < Cfg::FM; ++fm)
        a[fm] = *(const bf16x8*)(As + (arow + fm * 32) * Cfg::AP + kk * 16 + akof);
#pragma unroll
      for (int fn = 0; fn < Cfg::FN; ++fn) {
        const uint16_t* p = Bs + (kk * 16 + bk) * Cfg::BP + bn + fn * 32;
        i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
        i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * Cfg::BP));
        i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        b[fn] = __builtin_bit_cast(bf16x8, v);
      }
#pragma unroll
      for (int fm = 0; fm < Cfg::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < Cfg::FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[fm], b[fn], acc[fm][fn], 0, 0, 0);
    }
  }

  // Full K loop of one tile; lds holds two stages of Cfg::STAGE elements.
  __device__ __forceinline__ void run(const uint16_t* __restrict__ A,
                                      const uint16_t* __restrict__ B, int64_t M, int64_t N,
                                      int64_t K, int64_t m0, int64_t n0, uint16_t* lds) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
#pragma unroll
    for (int fm = 0; fm < Cfg::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < Cfg::FN; ++fn)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[fm][fn][i] = 0.0f;
    const int KT = (int)((K + Cfg::BK - 1) / Cfg::BK);
    if (KT == 0) return;
    load_global(A, B, M, N, K, m0, n0, 0, tid);
    store_lds(lds, tid);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      uint16_t* cur = lds + (kt & 1) * Cfg::STAGE;
      uint16_t* nxt = lds + ((kt + 1) & 1) * Cfg::STAGE;
      const bool more = kt + 1 < KT;
      if (more) load_global(A, B, M, N, K, m0, n0, (int64_t)(kt + 1) * Cfg::BK, tid);
      mma_stage(cur, wave, lane);
      if (more) store_lds(nxt, tid);
      __syncthreads();
    }
  }

  // Store the fp32 tile into P[M][N] (row-major). Accumulator layout of the
  // 32x32 block: lane l holds column l%32, rows 8*(i/4) + 4*(l/32) + i%4.
  __device__ __forceinline__ void store_partial(float* __restrict__ P, int64_t M, int64_t N,
                                                int64_t m0, int64_t n0) const {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int fm = 0; fm < Cfg::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < Cfg::FN; ++fn) {
        int64_t col = n0 + wn * Cfg::WN + fn * 32 + (lane & 31);
        int64_t rbase = m0 + wm * Cfg::WM + fm * 32 + (lane >> 5) * 4;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          int64_t row = rbase + (i >> 2) * 8 + (i & 3);
          if (row < M && col < N) P[row * N + col] = acc[fm][fn][i];
        }
      }
  }
};

// ----------------------------------------------------------------- reduce

// Peer element access: 8 consecutive values starting at element offset e.
template <typename PT>
struct PeerLoad;
template <>
struct PeerLoad<uint16_t> {  // bfloat16 peers: one 16-byte load
  u32x4 v;
  __device__ __forceinline__ void load(const uint16_t* p, int64_t e) {
    v = __builtin_nontemporal_load((const u32x4*)(p + e));
  }
  __device__ __forceinline__ void add_to(float* acc) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += bf16_lo(v[i]);
      acc[2 * i + 1] += bf16_hi(v[i]);
    }
  }
};
template <>
struct PeerLoad<float> {  // float32 peers: two 16-byte loads
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p, int64_t e) {
    a = __builtin_nontemporal_load((const f32x4*)(p + e));
    b = __builtin_nontemporal_load((const f32x4*)(p + e + 4));
  }
  __device__ __forceinline__ void add_to(float* acc) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[i] += a[i];
      acc[4 + i] += b[i];
    }
  }
};

template <typename CT>
__device__ __forceinline__ void store_c(CT* C, int64_t e, const float* acc);
template <>
__device__ __forceinline__ void store_c<uint16_t>(uint16_t* C, int64_t e, const float* acc) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = f32_to_bf16_rne(acc[2 * i]) | (f32_to_bf16_rne(acc[2 * i + 1]) << 16);
  __builtin_nontemporal_store(o, (u32x4*)(C + e));
}
template <>
__device__ __forceinline__ void store_c<float>(float* C, int64_t e, const float* acc) {
  f32x4 a = {acc[0], acc[1], acc[2], acc[3]}, b = {acc[4], acc[5], acc[6], acc[7]};
  __builtin_nontemporal_store(a, (f32x4*)(C + e));
  __builtin_nontemporal_store(b, (f32x4*)(C + e + 4));
}

// Sum for CH chunks of 8 elements at element offsets e[0..CH-1]:
//   C = (((P + peer_0) + peer_1) + ... + peer_{n-1}), float32, then rounded once.
// Peers are fetched in batches of 8 (indices past the last peer re-read the last
// peer and are not added), so that many loads are in flight before the adds.
template <int CH, typename PT, typename CT>
__device__ __forceinline__ void reduce_chunks(const float* __restrict__ P,
                                              const PT* __restrict__ peers, int n_peers,
                                              int64_t peer_stride, CT* __restrict__ C,
                                              const int64_t* e) {
  float acc[CH][8];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    f32x4 a = *(const f32x4*)(P + e[c]);
    f32x4 b = *(const f32x4*)(P + e[c] + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[c][i] = a[i];
      acc[c][4 + i] = b[i];
    }
  }
  constexpr int PB = 8;
  for (int p0 = 0; p0 < n_peers; p0 += PB) {
    PeerLoad<PT> v[CH][PB];
#pragma unroll
    for (int s = 0; s < PB; ++s) {
      int p = p0 + s < n_peers ? p0 + s : n_peers - 1;
#pragma unroll
      for (int c = 0; c < CH; ++c) v[c][s].load(peers + (int64_t)p * peer_stride, e[c]);
    }
#pragma unroll
    for (int s = 0; s < PB; ++s) {
      if (p0 + s < n_peers) {
#pragma unroll
        for (int c = 0; c < CH; ++c) v[c][s].add_to(acc[c]);
      }
    }
  }
#pragma unroll
  for (int c = 0; c < CH; ++c) store_c<CT>(C, e[c], acc[c]);
}

// Reduce the region rows [m0, m0+rows) x cols [n0, n0+cols) of an M x N output;
// cols is a multiple of 8. All 256 threads of the workgroup take part.
template <typename PT, typename CT>
__device__ __forceinline__ void reduce_region(const float* __restrict__ P,
                                              const PT* __restrict__ peers, int n_peers,
                                              CT* __restrict__ C, int64_t M, int64_t N, int64_t m0,
                                              int64_t n0, int rows, int cols) {
  const int cpr = cols >> 3;
  const int total = rows * cpr;
  const int64_t stride = M * N;
  constexpr int CH = 2;
  int q = threadIdx.x;
  for (; q + (CH - 1) * kThreads < total; q += CH * kThreads) {
    int64_t e[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      int qq = q + c * kThreads;
      e[c] = (m0 + qq / cpr) * N + n0 + (qq % cpr) * 8;
    }
    reduce_chunks<CH, PT, CT>(P, peers, n_peers, stride, C, e);
  }
  for (; q < total; q += kThreads) {
    int64_t e[1] = {(m0 + q / cpr) * N + n0 + (q % cpr) * 8};
    reduce_chunks<1, PT, CT>(P, peers, n_peers, stride, C, e);
  }
}

}  // namespace mk
