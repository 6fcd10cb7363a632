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

#include "mk_kernels.h"

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
// Branch-free (a select), so it never splits the surrounding code into blocks.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rounded = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  const uint32_t quiet = (u >> 16) | 0x40u;
  return (u & 0x7FFFFFFFu) > 0x7F800000u ? quiet : rounded;
}

// ----------------------------------------------------------------- timers, flags

// Constant 100 MHz clock shared by all compute units.
__device__ __forceinline__ uint64_t ticks() { return __builtin_amdgcn_s_memrealtime(); }

// Readiness flags (Figure 2, item 1: compute blocks write completed tiles to GPU
// memory and set readiness flags; Table 2's caption: completion of a transfer and
// its visibility in GPU memory are separate requirements).
//
// Every tile is produced and consumed by workgroups of the same XCD (tiles are
// queued per XCD), and the XCD's L2 is the point where all of its compute units
// see the same data (the per-CU vector L1 is write-through). So:
//   producer: each wave waits until its partial-tile stores are acknowledged by
//             the L2 (vmcnt = 0), the workgroup meets at a barrier, then one lane
//             stores the flag with an agent-scope atomic (no L2 write-back);
//   consumer: one lane polls the flag with agent-scope atomic loads; the
//             partial is then read from the L2 unless the compute unit's L1
//             already holds a copy of one of its lines. With N a multiple of 32
//             floats every 128-byte line of the partial belongs to one reduce
//             unit, read once per call, so no copy can exist (the L1 starts
//             each kernel empty) and nothing is invalidated. Otherwise the
//             consumer acquires at agent scope (buffer_inv sc1), which
//             invalidates its L1; the workgroup then meets at a barrier.
// Measured with the hand-off litmus (mk_flag_handoff), which rereads one word:
// producer as above with the agent-scope acquire carried the data in every one
// of 200,000 same-XCD hand-offs; a workgroup-scope invalidate (buffer_inv sc0,
// inv_group_scope below) in its place left the L1's copy in use (199,999 stale
// reads). The acquire costs the 4096x8192x1792 call about 20 us when used on
// every reduce unit, hence its restriction to shared lines. Across XCDs the
// producer's L2 must be written back too: the agent-scope variant (release and
// acquire) is kept for that.
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup-scope cache invalidate. Not a consumer acquire: it does not refresh
// a line the compute unit's L1 already holds (see above); only the hand-off
// litmus uses it, to show that.
__device__ __forceinline__ void inv_group_scope() {
  asm volatile("buffer_inv sc0\n\ts_waitcnt vmcnt(0)" ::: "memory");
}

__device__ __forceinline__ void store_flag(int* flag, int v) {
  __hip_atomic_store(flag, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void publish_flag_agent(int* flag, int epoch) {
  __hip_atomic_store(flag, epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int load_relaxed(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void acquire_fence_agent() {
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// Hardware id of the XCD this wave runs on.
__device__ __forceinline__ int xcc_id() {
  unsigned x;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
  return (int)(x & 0xF);
}

// Sleep for about n * 512 cycles (s_sleep takes an immediate).
__device__ __forceinline__ void backoff_sleep(int n) {
  for (int i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(8);
}

// ----------------------------------------------------------------- tile GEMM

typedef __attribute__((address_space(3))) char lds_char;

// One 16-byte-per-lane direct load into LDS: lane i's 16 bytes from g land at
// LDS byte address lds + 16*i (global_load_lds_dwordx4, LDS base in M0).
// Issued through inline asm so that the compiler does not treat the pending LDS
// write as aliasing every later LDS read (it would then wait for all
// outstanding loads before each stage and undo the prefetch). The caller orders
// the writes with explicit vmcnt waits and barriers; loads complete in issue
// order, so the compiler's own vmcnt waits stay correct.
__device__ __forceinline__ void dma16(const void* g, const char* lds) {
  unsigned a = __builtin_amdgcn_readfirstlane((unsigned)(size_t)(const lds_char*)lds);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(a) : "memory");
}

// Tile shape: BM x BN outputs per workgroup, BK k-values per stage, NS stages in
// LDS: 32 x 4 (three stages of loads in flight while one is computed; one stage
// per CU was latency-bound) or 64 x 2 (the same LDS bytes in half as many
// barriers; measured 5-7% faster on 256 x 256 tiles). Four waves in a 2 x 2 arrangement; each wave
// owns a (BM/2) x (BN/2) block made of 32 x 32 matrix-core blocks
// (v_mfma_f32_32x32x16_bf16, 32 cycles each).
//
// LDS holds the tiles unpadded and XOR-swizzled in 16-byte chunks so that
// (a) global_load_lds_dwordx4 can fill them (it writes a wave's 64 x 16 bytes to
//     consecutive LDS addresses; the swizzle is applied on the global side), and
// (b) the fragment reads hit distinct banks (64 banks of 4 bytes):
//   A tile [BM][BK]: 64-byte rows (BK 32), chunk c of row r stored at
//     c ^ ((r >> 2) & 3), or 128-byte rows (BK 64) at c ^ ((r >> 1) & 7);
//     a 16-lane phase of ds_read_b128 covers rows r..r+15 of one chunk column.
//   B tile [BK][BN]: chunk c of row k stored at c ^ (4 * (k & 3)) (2 * (k & 3)
//     for 64-wide tiles, whose rows hold 8 chunks); the gfx950 transposing read
//     (ds_read_b64_tr_b16) has 16 lanes read a 4(k) x 16(n) block, so 32 lanes
//     touch 4 rows x 4 chunks = all 64 banks once.
// Default gate of GemmTile::run: every k-tile's inputs are already in memory.
struct NoGate {
  __device__ __forceinline__ void operator()(int) const {}
};

// NW waves per workgroup, WGN of them along N (4 and 2: a 2 x 2 grid of wave
// tiles; 8 and 4: a 2 x 4 grid)
template <int BM_, int BN_, int BK_ = 32, int NS_ = 4, int NW_ = 4, int WGN_ = 2>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, NS = NS_;
  static constexpr int NW = NW_, WGN = WGN_;
  // A tile rows are BK*2 bytes: chunk c of row r is stored at c ^ a_swz(r), so
  // that 16 consecutive rows of one chunk column hit distinct 16-byte bank groups
  static constexpr int A_CPR = BK * 2 / 16;  // 16-byte chunks per A row (4 or 8)
  __device__ __forceinline__ static int a_swz(int row) {
    return A_CPR == 4 ? (row >> 2) & 3 : (row >> 1) & 7;
  }
  // B tile rows are BN*2 bytes: chunk c of row k is stored at c ^ b_swz(k), which
  // stays inside the row (16 or more chunks: 4 * (k & 3); 8 chunks, 64-wide
  // tiles: 2 * (k & 3))
  static constexpr int B_CPR = BN * 2 / 16;
  __device__ __forceinline__ static int b_swz(int row) {
    return B_CPR >= 16 ? 4 * (row & 3) : 2 * (row & 3);
  }
  // fused kernel: workgroups per CU
  static constexpr int OCC = BM * BN >= 256 * 256 ? 1 : 2;
  // fused kernel: a tile's reduce is split into RSPLIT row slabs, each claimed
  // on its own, so that the last reduces spread over every idle workgroup
  static constexpr int RSPLIT = BM / 64;
  static constexpr int KSTEPS = BK / 16;
  static constexpr int WM = BM / (NW / WGN), WN = BN / WGN;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int A_ROW = BK * 2;              // bytes per A row
  static constexpr int A_BYTES = BM * A_ROW;
  static constexpr int B_ROW = BN * 2;              // bytes per B row
  static constexpr int B_BYTES = BK * B_ROW;
  static constexpr int STAGE = A_BYTES + B_BYTES;   // bytes per stage
  static constexpr int LDS_BYTES = NS * STAGE;
  static constexpr int A_LD = A_BYTES / 1024 / NW;  // 1 KiB direct loads per wave
  static constexpr int B_LD = B_BYTES / 1024 / NW;
  static constexpr int LD = A_LD + B_LD;            // direct loads per wave per stage
  static constexpr int A_ROWS_PER_LD = 1024 / A_ROW;
  static constexpr int B_ROWS_PER_LD = 1024 / B_ROW;
  static_assert(FM >= 1 && FN >= 1 && FN <= 4, "tile shape");
  static_assert(A_LD >= 1 && B_LD >= 1 && B_ROW <= 1024, "tile too small for its waves");
  static_assert(NW / WGN == 2, "two rows of wave tiles");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// Tile index -> (tile row, tile column), grouped so that consecutive tiles share
// A row-panels (GROUP rows of tiles sweep the columns together).
template <int GROUP = 8>
__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  int group_size = GROUP * tiles_n;
  int g = t / group_size;
  int first = g * GROUP;
  int gm = tiles_m - first < GROUP ? tiles_m - first : GROUP;
  int w = t - g * group_size;
  tm = first + w % gm;
  tn = w / gm;
}

// Fused kernel's map: tile_coords, then a column permutation that sends each run
// of tiles_n/4 consecutive tile columns to every 4th column. An XCD's share of
// tiles (a contiguous range of t) keeps the same number of A and B panels for
// L2 reuse, but its tiles no longer sit side by side in memory: concurrent
// streams spread over the whole row of every operand, which measured 10-25%
// more reduce bandwidth than compact blocks of tiles per XCD.
template <int GROUP = 8>
__device__ __forceinline__ void fused_tile_coords(int t, int tiles_m, int tiles_n, int& tm,
                                                  int& tn) {
  tile_coords<GROUP>(t, tiles_m, tiles_n, tm, tn);
  constexpr int S = 4;
  if (tiles_n >= 2 * S && tiles_n % S == 0) {
    const int w = tiles_n / S;
    tn = (tn % w) * S + tn / w;
  }
}

// GEMM+ReduceScatter order: each XCD's queue (local index i of cnt, first
// global index q0) starts with its share [ox0, ox0 + ox) of the tiles in the
// tile rows that hold owned rows, [tmo0, tmo1), so that their reduce overlaps
// the other tiles' GEMMs rather than ending the kernel; the other tiles follow.
// Both groups keep the grouped order of tile_coords.
__device__ __forceinline__ void rs_tile_coords(int i, int q0, int ox0, int ox, int tiles_m,
                                               int tiles_n, int tmo0, int tmo1, int& tm,
                                               int& tn) {
  const int h = tmo1 - tmo0;
  if (i < ox) {
    tile_coords(ox0 + i, h, tiles_n, tm, tn);
    tm += tmo0;
  } else {
    tile_coords(q0 - ox0 + (i - ox), tiles_m - h, tiles_n, tm, tn);
    if (tm >= tmo0) tm += h;
  }
}
// XCD x's share of the n_ot tiles with owned rows: at most ceil(n_ot / n_xcd)
// and at most its queue, in XCD order, so that every one of them is placed.
__device__ __forceinline__ void rs_share(int x, int n_xcd, int T, int n_ot, int& ox0, int& ox) {
  const int q = (n_ot + n_xcd - 1) / n_xcd;
  int acc = 0, o = 0;
  for (int y = 0; y <= x; ++y) {
    const int cnt = (int)(((int64_t)(y + 1) * T) / n_xcd - ((int64_t)y * T) / n_xcd);
    int v = cnt < q ? cnt : q;
    v = v < n_ot - acc ? v : n_ot - acc;
    v = v > 0 ? v : 0;
    if (y == x) o = v;
    else acc += v;
  }
  ox0 = acc;
  ox = o;
}

template <class Cfg>
struct GemmTile {
  f32x16 acc[Cfg::FM][Cfg::FN];

  // Per-lane global element offsets of this wave's 16-byte chunks of a stage,
  // before the k offset. Rows beyond M and columns beyond N are clamped to the
  // last valid one: they only feed outputs that are never stored.
  struct Src {
    int64_t a[Cfg::A_LD];
    int64_t b[Cfg::B_LD];
  };

  // lda: A's row pitch in elements (K when A holds just the k-range multiplied).
  __device__ __forceinline__ static void sources(Src& s, int64_t M, int64_t N, int64_t lda,
                                                 int64_t m0, int64_t n0, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < Cfg::A_LD; ++i) {
      int blk = wave * Cfg::A_LD + i;
      int byte = lane * 16;
      int row = blk * Cfg::A_ROWS_PER_LD + byte / Cfg::A_ROW;
      int p = (byte % Cfg::A_ROW) / 16;
      int c = p ^ Cfg::a_swz(row);
      int64_t gm = m0 + row < M ? m0 + row : M - 1;
      s.a[i] = gm * lda + c * 8;
    }
#pragma unroll
    for (int i = 0; i < Cfg::B_LD; ++i) {
      int blk = wave * Cfg::B_LD + i;
      int byte = lane * 16;
      int row = blk * Cfg::B_ROWS_PER_LD + byte / Cfg::B_ROW;
      int p = (byte % Cfg::B_ROW) / 16;
      int c = p ^ Cfg::b_swz(row);
      int64_t gn = n0 + c * 8 < N ? n0 + c * 8 : N - 8;
      s.b[i] = (int64_t)row * N + gn;
    }
  }

  // Full k-tile [k0, k0+BK) straight into LDS (no register staging).
  __device__ __forceinline__ static void load_direct(const Src& s, const uint16_t* __restrict__ A,
                                                     const uint16_t* __restrict__ B, int64_t N,
                                                     int64_t k0, char* stage, int wave) {
#pragma unroll
    for (int i = 0; i < Cfg::A_LD; ++i)
      dma16(A + s.a[i] + k0, stage + (wave * Cfg::A_LD + i) * 1024);
#pragma unroll
    for (int i = 0; i < Cfg::B_LD; ++i)
      dma16(B + s.b[i] + k0 * N, stage + Cfg::A_BYTES + (wave * Cfg::B_LD + i) * 1024);
  }

  // Last, partial k-tile: same LDS image, but k >= K reads as zero; used at most
  // once per tile, when K is not a multiple of BK. K is a multiple of 8, so each
  // 16-byte chunk lies wholly below K (loaded straight into LDS, like a full
  // stage) or wholly at or past K (zero-filled by an LDS store). No load here is
  // one the compiler tracks, so the k-loop around it carries no extra waits.
  __device__ __forceinline__ static void load_guarded(const Src& s, const uint16_t* __restrict__ A,
                                                      const uint16_t* __restrict__ B, int64_t N,
                                                      int64_t K, int64_t k0, char* stage, int wave,
                                                      int lane) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < Cfg::A_LD; ++i) {
      int byte = lane * 16;
      int row = (wave * Cfg::A_LD + i) * Cfg::A_ROWS_PER_LD + byte / Cfg::A_ROW;
      int c = ((byte % Cfg::A_ROW) / 16) ^ Cfg::a_swz(row);
      char* dst = stage + (wave * Cfg::A_LD + i) * 1024;
      if (k0 + c * 8 < K) dma16(A + s.a[i] + k0, dst);
      else *(u32x4*)(dst + lane * 16) = zero;
    }
#pragma unroll
    for (int i = 0; i < Cfg::B_LD; ++i) {
      int row = (wave * Cfg::B_LD + i) * Cfg::B_ROWS_PER_LD + (lane * 16) / Cfg::B_ROW;
      char* dst = stage + Cfg::A_BYTES + (wave * Cfg::B_LD + i) * 1024;
      if (k0 + row < K) dma16(B + s.b[i] + k0 * N, dst);
      else *(u32x4*)(dst + lane * 16) = zero;
    }
    wait_loads(0);
  }

  // Fragment addresses within a stage (bytes), per lane.
  struct Frag {
    int a[Cfg::KSTEPS];    // A offset for step kk (row and swizzled chunk)
    int b[Cfg::FN];        // B offset for step 0, low half (step kk adds 16 rows)
  };

  __device__ __forceinline__ static void frag_offsets(Frag& f, int wave, int lane) {
    const int wm = wave / Cfg::WGN, wn = wave % Cfg::WGN;
    const int arow = wm * Cfg::WM + (lane & 31);  // + 32*fm keeps a_swz(row)
#pragma unroll
    for (int kk = 0; kk < Cfg::KSTEPS; ++kk) {
      int c = 2 * kk + (lane >> 5);
      f.a[kk] = arow * Cfg::A_ROW + ((c ^ Cfg::a_swz(arow)) * 16);
    }
    const int g = lane >> 4, r = lane & 15;
    const int brow = (g >> 1) * 8 + (r >> 2);  // + 16*kk (+4 for the high half)
#pragma unroll
    for (int fn = 0; fn < Cfg::FN; ++fn) {
      int c = (wn * Cfg::WN + fn * 32) / 8 + (g & 1) * 2 + ((r & 3) >> 1);
      int p = c ^ Cfg::b_swz(brow);
      f.b[fn] = Cfg::A_BYTES + brow * Cfg::B_ROW + p * 16 + (r & 1) * 8;
    }
  }

  __device__ __forceinline__ static void read_frags(const char* stage, const Frag& f, int kk,
                                                    bf16x8 (&a)[Cfg::FM], bf16x8 (&b)[Cfg::FN]) {
#pragma unroll
    for (int fm = 0; fm < Cfg::FM; ++fm)
      a[fm] = *(const bf16x8*)(stage + f.a[kk] + fm * 32 * Cfg::A_ROW);
#pragma unroll
    for (int fn = 0; fn < Cfg::FN; ++fn) {
      const char* p = stage + f.b[fn] + kk * 16 * Cfg::B_ROW;
      i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
      i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * Cfg::B_ROW));
      b[fn] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  }

  __device__ __forceinline__ void mma(const bf16x8 (&a)[Cfg::FM], const bf16x8 (&b)[Cfg::FN]) {
#pragma unroll
    for (int fm = 0; fm < Cfg::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < Cfg::FN; ++fn)
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[fm], b[fn], acc[fm][fn], 0, 0, 0);
  }

  // NM MFMAs, each followed by up to RPM of the LEFT remaining LDS reads.
  template <int NM, int RPM, int LEFT>
  __device__ __forceinline__ static void interleave() {
    if constexpr (NM > 0) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      constexpr int n = LEFT < RPM ? LEFT : RPM;
      if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(0x100, n, 0);
      interleave<NM - 1, RPM, LEFT - n>();
    }
  }

  // One stage: KSTEPS steps of k = 16. The fragments of step kk+1 are read from
  // LDS while the matrix cores work on step kk; each step is its own scheduling
  // region (its MFMAs are independent of each other) and the group barriers pin
  // one LDS read between consecutive MFMAs, so LDS latency hides behind MFMAs.
  __device__ __forceinline__ void compute_stage(const char* stage, const Frag& f) {
    constexpr int NR = Cfg::FM + 2 * Cfg::FN;  // LDS reads per step
    constexpr int NM = Cfg::FM * Cfg::FN;      // MFMAs per step
    constexpr int RPM = (NR + NM - 1) / NM;
    bf16x8 a[2][Cfg::FM], b[2][Cfg::FN];
    read_frags(stage, f, 0, a[0], b[0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < Cfg::KSTEPS; ++kk) {
      if (kk + 1 < Cfg::KSTEPS) read_frags(stage, f, kk + 1, a[(kk + 1) & 1], b[(kk + 1) & 1]);
      mma(a[kk & 1], b[kk & 1]);
      if (kk + 1 < Cfg::KSTEPS) interleave<NM, RPM, NR>();
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Wait until at most n of this wave's loads are outstanding (n is a multiple of
  // LD, 0 .. (NS-2)*LD: the direct loads of the later stages in flight).
  template <int I = Cfg::NS - 2>
  __device__ __forceinline__ static void wait_loads(int n) {
    if constexpr (I <= 0) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
      if (n >= I * Cfg::LD) asm volatile("s_waitcnt vmcnt(%0)" ::"i"(I * Cfg::LD) : "memory");
      else wait_loads<I - 1>(n);
    }
  }

  // Full K loop of one tile. Stage kt lives in LDS slot kt % NS; loads for
  // stages kt+1 .. kt+NS-1 are in flight while stage kt is computed.
  // gate(kt) runs in every lane before the loads of k-tile kt are issued (a
  // consumer that waits for its inputs to arrive); NoGate does nothing.
  // lda: A's row pitch (0 = K); a k-range [k0, k0+K) of a wider product is run
  // with A and B advanced to k0 and lda the full width.
  template <class Gate = NoGate>
  __device__ __forceinline__ void run(const uint16_t* __restrict__ A,
                                      const uint16_t* __restrict__ B, int64_t M, int64_t N,
                                      int64_t K, int64_t m0, int64_t n0, char* lds,
                                      Gate gate = Gate(), int64_t lda = 0) {
    static_assert(Cfg::NS >= 2 && (Cfg::NS - 2) * Cfg::LD <= 63, "vmcnt counts at most 63 loads");
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
#pragma unroll
    for (int fm = 0; fm < Cfg::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < Cfg::FN; ++fn)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[fm][fn][i] = 0.0f;
    const int KT = (int)((K + Cfg::BK - 1) / Cfg::BK);
    if (KT == 0) return;
    const int KF = (int)(K / Cfg::BK);  // full k-tiles; tile KF (if < KT) is partial
    Src s;
    sources(s, M, N, lda > 0 ? lda : K, m0, n0, wave, lane);
    Frag f;
    frag_offsets(f, wave, lane);
    // Prologue: stages 0 .. NS-2. The partial tile, if any, is the last stage
    // and is loaded through registers when its turn comes.
#pragma unroll
    for (int j = 0; j < Cfg::NS - 1; ++j)
      if (j < KF) {
        gate(j);
        load_direct(s, A, B, N, (int64_t)j * Cfg::BK, lds + j * Cfg::STAGE, wave);
      }
    for (int kt = 0; kt < KT; ++kt) {
      char* cur = lds + (kt % Cfg::NS) * Cfg::STAGE;
      if (kt == KF) {
        // partial tile: loaded now (the slot was freed by the previous barrier)
        gate(kt);
        load_guarded(s, A, B, N, K, (int64_t)kt * Cfg::BK, cur, wave, lane);
      } else {
        // direct loads of the full stages after kt that are already issued
        int later = KF - 1 - kt;
        later = later < Cfg::NS - 2 ? later : Cfg::NS - 2;
        wait_loads(later * Cfg::LD);
      }
      __syncthreads();  // stage kt complete in LDS; slot (kt-1) % NS is free
      const int kn = kt + Cfg::NS - 1;
      if (kn < KF) {
        gate(kn);
        load_direct(s, A, B, N, (int64_t)kn * Cfg::BK, lds + (kn % Cfg::NS) * Cfg::STAGE, wave);
      }
      compute_stage(cur, f);
    }
    __syncthreads();  // every wave is done with LDS before it is reused
  }

  // Store the fp32 tile into P[M][N] (row-major). Accumulator layout of the
  // 32x32 block: lane l holds column l%32, rows 8*(i/4) + 4*(l/32) + i%4.
  __device__ __forceinline__ void store_partial(float* __restrict__ P, int64_t M, int64_t N,
                                                int64_t m0, int64_t n0) const {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave / Cfg::WGN, wn = wave % Cfg::WGN;
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

  // In-place reduce of a tile: the fp32 accumulators go through LDS (BN floats
  // per row) in NPASS passes. Pass p takes accumulator blocks fm in
  // [p*FM/NPASS, (p+1)*FM/NPASS) of every wave, i.e. for each wave row wm the
  // band of BAND tile rows starting at wm*WM + p*BAND; the two bands sit one
  // after the other in LDS. Blocks of later passes stay in registers meanwhile
  // (at most half of them), so the reduce that follows has room.
  static constexpr int LDS_ROWS = Cfg::LDS_BYTES / (Cfg::BN * 4);
  // one pass when the whole fp32 tile fits the LDS (small tiles)
  static constexpr int NPASS = Cfg::BM <= LDS_ROWS ? 1 : Cfg::BM / LDS_ROWS;
  static constexpr int BAND = Cfg::WM / NPASS;
  static_assert(NPASS >= 1 && (NPASS == 1 || Cfg::BM % LDS_ROWS == 0) && Cfg::FM % NPASS == 0,
                "LDS passes");
  static_assert(2 * BAND <= LDS_ROWS, "two bands of wave rows per pass");

  // Lanes 0-31 and 32-63 each write 128 contiguous bytes per store, which
  // touches every bank once.
  template <int PASS>
  __device__ __forceinline__ void stage_pass_lds(char* lds) const {
    typedef __attribute__((address_space(3))) float lds_float;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave / Cfg::WGN, wn = wave % Cfg::WGN;
    lds_float* f = (lds_float*)(lds_char*)lds;
    constexpr int F0 = PASS * Cfg::FM / NPASS, F1 = (PASS + 1) * Cfg::FM / NPASS;
#pragma unroll
    for (int fm = F0; fm < F1; ++fm)
#pragma unroll
      for (int fn = 0; fn < Cfg::FN; ++fn) {
        const int col = wn * Cfg::WN + fn * 32 + (lane & 31);
        const int rbase = wm * BAND + (fm - F0) * 32 + (lane >> 5) * 4;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          f[(rbase + (i >> 2) * 8 + (i & 3)) * Cfg::BN + col] = acc[fm][fn][i];
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
  __device__ __forceinline__ void load(const uint16_t* p) {
    v = __builtin_nontemporal_load((const u32x4*)p);
  }
  // acc[j] = peer[j], j = 0..7: each bfloat16 half widened exactly
  __device__ __forceinline__ void set(float* acc) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = bf16_lo(v[i]);
      acc[2 * i + 1] = bf16_hi(v[i]);
    }
  }
  // acc[j] += peer[j]: widen exactly, then one correctly rounded fp32 add
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
  __device__ __forceinline__ void load(const float* p) {
    a = __builtin_nontemporal_load((const f32x4*)p);
    b = __builtin_nontemporal_load((const f32x4*)(p + 4));
  }
  __device__ __forceinline__ void set(float* acc) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[i] = a[i];
      acc[4 + i] = b[i];
    }
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

// Every path sums the same way, element by element, in float32:
//   C = round((((peer_0 + peer_1) + ...) + peer_{n-1}) + P)
// (C = round(P) without peers): the peers in index order, then the local
// partial P. Reducer counts, the controller, tiles reduced in place or handed
// over, peers summed ahead of the partial, and the two-kernel baseline all give
// the same bits. Since the partial comes last, a reducer can sum a tile's peers
// before the tile's GEMM has finished.

// Generic path (any peer count): CH chunks of 8 elements at offsets e[], peers
// fetched in batches (8 bfloat16 or 4 float32 peers) so that many loads are in
// flight before the adds.
template <int CH, typename PT, typename CT>
__device__ __forceinline__ void reduce_chunks(const float* __restrict__ P,
                                              const PT* __restrict__ peers, int n_peers,
                                              int64_t peer_stride, CT* __restrict__ C,
                                              const int64_t* e) {
  float acc[CH][8];
  f32x4 pa[CH], pb[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    pa[c] = *(const f32x4*)(P + e[c]);
    pb[c] = *(const f32x4*)(P + e[c] + 4);
  }
  constexpr int PB = sizeof(PT) == 2 ? 8 : 4;
  for (int p0 = 0; p0 < n_peers; p0 += PB) {
    PeerLoad<PT> v[CH][PB];
#pragma unroll
    for (int s = 0; s < PB; ++s) {
      if (p0 + s < n_peers) {
#pragma unroll
        for (int c = 0; c < CH; ++c) v[c][s].load(peers + (int64_t)(p0 + s) * peer_stride + e[c]);
      }
    }
#pragma unroll
    for (int s = 0; s < PB; ++s) {
      if (p0 + s < n_peers) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          if (s == 0 && p0 == 0) v[c][s].set(acc[c]);
          else v[c][s].add_to(acc[c]);
        }
      }
    }
  }
#pragma unroll
  for (int c = 0; c < CH; ++c) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[c][i] = n_peers > 0 ? acc[c][i] + pa[c][i] : pa[c][i];
      acc[c][4 + i] = n_peers > 0 ? acc[c][4 + i] + pb[c][i] : pb[c][i];
    }
    store_c<CT>(C, e[c], acc[c]);
  }
}

// Ring path (NP >= 1 peers known at compile time). Thread t handles chunks t,
// t+256, ... of a tile region. A chunk's loads (its NP peer vectors, and its
// fp32 partial when the sum ends with one) are issued together, DEPTH-1 chunks
// ahead of the chunk being summed. Vector memory loads complete in issue order,
// so waiting for a chunk's loads waits for nothing issued after them: while
// chunk q is summed the loads of the next DEPTH-1 chunks stay in flight. A
// reducer workgroup is the only one on its compute unit, so latency has to be
// covered by bytes in flight (at most 63 loads per wave) rather than by more
// waves.
//
// Addressing: every operand has a wave-uniform 64-bit base for the region (kept
// in scalar registers) and each lane one 32-bit element offset from it, which it
// advances by a fixed step per chunk without a division. A chunk index past the
// end is clamped to the last chunk: that lane reads the same inputs as the lane
// that owns the chunk and stores the same bits to the same place, so no lane
// needs a branch, and the loop runs on a wave-uniform bound.
//
// Where a chunk's fp32 partial comes from: the workspace in device memory, LDS
// (a tile reduced in place by the workgroup that computed it), or nowhere (peers
// summed ahead of their tile's partial). The first two give the same bits.
struct PartialGlobal {
  static constexpr bool kHas = true, kLate = false;
  const float* __restrict__ P;  // region base
  __device__ __forceinline__ void load(f32x4& a, f32x4& b, uint32_t off, uint32_t) const {
    const uint32_t op = off * 4u;
    a = *(const f32x4*)((const char*)P + op);
    b = *(const f32x4*)((const char*)P + op + 16u);
  }
};
// The partial of a product computed in NP k-parts of equal length: ((P_0 + P_1)
// + ...) + P_{NP-1} in float32, parts `stride` floats apart (the parts' sum is
// the tile's partial; it is formed before anything is added to it).
template <int NP>
struct PartialGlobalN {
  static constexpr bool kHas = true, kLate = false;
  const float* __restrict__ P;  // region base of part 0
  uint32_t stride_bytes;        // bytes between two parts' region bases
  __device__ __forceinline__ void load(f32x4& a, f32x4& b, uint32_t off, uint32_t) const {
    const uint32_t op = off * 4u;
    f32x4 va[NP], vb[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const char* base = (const char*)P + (size_t)p * stride_bytes;
      va[p] = *(const f32x4*)(base + op);
      vb[p] = *(const f32x4*)(base + op + 16u);
    }
    a = va[0];
    b = vb[0];
#pragma unroll
    for (int p = 1; p < NP; ++p)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = a[i] + va[p][i];
        b[i] = b[i] + vb[p][i];
      }
  }
};
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
struct PartialLds {
  static constexpr bool kHas = true, kLate = false;
  const lds_char* base;  // region base in LDS, rows of the LDS pitch
  __device__ __forceinline__ void load(f32x4& a, f32x4& b, uint32_t, uint32_t loff) const {
    a = *(const lds_f32x4*)(base + loff * 4u);
    b = *(const lds_f32x4*)(base + loff * 4u + 16u);
  }
};
// The same, read when the chunk is summed rather than with its peers' loads: a
// chunk in flight then holds only its peers' registers (the LDS read's latency
// hides behind the peer additions, which come first).
struct PartialLdsLate : PartialLds {
  static constexpr bool kLate = true;
};
struct NoPartial {
  static constexpr bool kHas = false, kLate = false;
  __device__ __forceinline__ void load(f32x4&, f32x4&, uint32_t, uint32_t) const {}
};

// Where a chunk's sum goes: the output in device memory (rounded to CT), or the
// float32 peer sum into LDS (row pitch of the LDS region).
template <typename CT>
struct OutC {
  CT* __restrict__ C;  // region base
  __device__ __forceinline__ void store(uint32_t off, uint32_t, const float* acc) const {
    store_c<CT>((CT*)((char*)C + off * (uint32_t)sizeof(CT)), 0, acc);
  }
};
struct OutLds {
  lds_char* base;
  __device__ __forceinline__ void store(uint32_t, uint32_t loff, const float* acc) const {
    const f32x4 a = {acc[0], acc[1], acc[2], acc[3]}, b = {acc[4], acc[5], acc[6], acc[7]};
    *(lds_f32x4*)(base + loff * 4u) = a;
    *(lds_f32x4*)(base + loff * 4u + 16u) = b;
  }
};

// sum = peer_0 + ... + peer_{NP-1} (+ partial), to OUT.
template <typename PT, int NP, typename PS, typename OUT>
struct SumOp {
  static_assert(NP >= 1, "ring sums have peers");
  PS ps;
  const PT* const __restrict__* peer;  // NP region bases
  OUT out;
  struct Chunk {
    f32x4 pa, pb;
    PeerLoad<PT> v[NP];
  };
  // Byte offsets are formed in 32 bits, so each load is a scalar base plus a
  // 32-bit vector offset.
  __device__ __forceinline__ void load(Chunk& k, uint32_t off, uint32_t loff) const {
    if constexpr (!PS::kLate) ps.load(k.pa, k.pb, off, loff);
    const uint32_t ov = off * (uint32_t)sizeof(PT);
#pragma unroll
    for (int s = 0; s < NP; ++s) k.v[s].load((const PT*)((const char*)peer[s] + ov));
    __builtin_amdgcn_sched_barrier(0);  // keep the group where the ring puts it
  }
  __device__ __forceinline__ void finish(const Chunk& k, uint32_t off, uint32_t loff) const {
    f32x4 pa = k.pa, pb = k.pb;
    if constexpr (PS::kLate) ps.load(pa, pb, off, loff);
    float acc[8];
    k.v[0].set(acc);
#pragma unroll
    for (int s = 1; s < NP; ++s) k.v[s].add_to(acc);
    if constexpr (PS::kHas) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] += pa[i];
        acc[4 + i] += pb[i];
      }
    }
    out.store(off, loff, acc);
    __builtin_amdgcn_sched_barrier(0);
  }
};

// sum = (peer sum left in LDS by a SumOp with NoPartial/OutLds) + partial, to
// C: the same float32 additions as one SumOp with the partial.
template <typename CT, typename PS = PartialGlobal>
struct PresumOp {
  PS ps;
  const lds_char* pre;  // region base in LDS
  OutC<CT> out;
  struct Chunk {
    f32x4 pa, pb;
  };
  __device__ __forceinline__ void load(Chunk& k, uint32_t off, uint32_t loff) const {
    ps.load(k.pa, k.pb, off, loff);
    __builtin_amdgcn_sched_barrier(0);
  }
  __device__ __forceinline__ void finish(const Chunk& k, uint32_t off, uint32_t loff) const {
    const f32x4 x = *(const lds_f32x4*)(pre + loff * 4u);
    const f32x4 y = *(const lds_f32x4*)(pre + loff * 4u + 16u);
    float acc[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[i] = x[i] + k.pa[i];
      acc[4 + i] = y[i] + k.pb[i];
    }
    out.store(off, loff, acc);
    __builtin_amdgcn_sched_barrier(0);
  }
};

// out = round(partial in LDS): a tile's rows published as they are (no peers).
template <typename OT>
struct CopyLdsOp {
  const lds_char* src;  // region base in LDS
  OutC<OT> out;
  struct Chunk {
    f32x4 a, b;
  };
  // the LDS reads run ahead of the stores, like a ring's loads
  __device__ __forceinline__ void load(Chunk& k, uint32_t, uint32_t loff) const {
    k.a = *(const lds_f32x4*)(src + loff * 4u);
    k.b = *(const lds_f32x4*)(src + loff * 4u + 16u);
    __builtin_amdgcn_sched_barrier(0);
  }
  __device__ __forceinline__ void finish(const Chunk& k, uint32_t off, uint32_t loff) const {
    const float acc[8] = {k.a[0], k.a[1], k.a[2], k.a[3], k.b[0], k.b[1], k.b[2], k.b[3]};
    out.store(off, loff, acc);
    __builtin_amdgcn_sched_barrier(0);
  }
};

// Walks chunk indices q = q0, q0+stride, ... (stride: the threads that share the
// region, 256 unless given) of a region of `cpr` chunks per row, giving each
// one's element offset for two row pitches (N for device memory, LP for a region
// in LDS), clamped to the last chunk past the end.
struct ChunkCursor {
  int q, c;                 // chunk index and its column chunk
  int stride;
  uint32_t off, loff;       // element offsets of chunk q (unclamped)
  int total, cpr;
  uint32_t last, llast;     // element offsets of the last chunk
  uint32_t step_off, step_loff;  // advance for 256 chunks without a row wrap
  int step_c;               // column-chunk advance for 256 chunks (256 % cpr)
  uint32_t wrap_off, wrap_loff;  // extra advance when the column wraps: pitch - 8 * cpr
  __device__ __forceinline__ void init(int q0, int total_, int cpr_, int64_t N, int64_t LP,
                                       int stride_ = kThreads) {
    stride = stride_;
    total = total_;
    cpr = cpr_;
    const int r = q0 / cpr_;
    c = q0 - r * cpr_;
    q = q0;
    off = (uint32_t)(r * N + c * 8);
    loff = (uint32_t)(r * LP + c * 8);
    const int rows = total_ / cpr_;
    last = (uint32_t)((rows - 1) * N + (cpr_ - 1) * 8);
    llast = (uint32_t)((rows - 1) * LP + (cpr_ - 1) * 8);
    const int a = stride_ / cpr_;
    step_c = stride_ - a * cpr_;
    step_off = (uint32_t)(a * N + step_c * 8);
    step_loff = (uint32_t)(a * LP + step_c * 8);
    wrap_off = (uint32_t)(N - 8 * cpr_);
    wrap_loff = (uint32_t)(LP - 8 * cpr_);
  }
  __device__ __forceinline__ uint32_t get() const { return q < total ? off : last; }
  __device__ __forceinline__ uint32_t lget() const { return q < total ? loff : llast; }
  __device__ __forceinline__ void advance() {
    q += stride;
    c += step_c;
    off += step_off;
    loff += step_loff;
    const bool wrap = c >= cpr;
    c = wrap ? c - cpr : c;
    off = wrap ? off + wrap_off : off;
    loff = wrap ? loff + wrap_loff : loff;
  }
};

template <int DEPTH, typename OP>
struct ReduceRing {
  // The workgroup's 256 threads walk the region's chunks together.
  __device__ __forceinline__ static void run(const OP& op, int total, int cpr, int64_t N,
                                             int64_t LP) {
    run_strided(op, total, cpr, N, LP, (int)threadIdx.x, kThreads);
  }
  // Thread t takes chunks t, t + stride, ... (stride a multiple of 64; the 64
  // lanes of a wave hold consecutive t).
  __device__ __forceinline__ static void run_strided(const OP& op, int total, int cpr, int64_t N,
                                                     int64_t LP, int t, int stride) {
    // loop bound on the wave's first chunk: a uniform (scalar) loop
    const int w0 = __builtin_amdgcn_readfirstlane(t & ~63);
    ChunkCursor ld, st;  // the chunk loaded next, the chunk summed next
    ld.init(t, total, cpr, N, LP, stride);
    st = ld;
    typename OP::Chunk b[DEPTH];
#pragma unroll
    for (int i = 0; i < DEPTH - 1; ++i) {
      op.load(b[i], ld.get(), ld.lget());
      ld.advance();
    }
    // At least one pass, so that no guard separates the loads above from the
    // loop (a wave whose chunks all lie past the end re-stores the last chunk).
    int k = 0;
    do {
#pragma unroll
      for (int i = 0; i < DEPTH; ++i) {
        op.load(b[(i + DEPTH - 1) % DEPTH], ld.get(), ld.lget());
        ld.advance();
        op.finish(b[i], st.get(), st.lget());
        st.advance();
      }
      k += DEPTH * stride;
    } while (w0 + k < total);
    // The last pass issued loads of clamped chunks that are never summed (L2
    // hits); the compute path waits for them before its GEMM loop.
  }
};

// The ring of the streaming waves of a wave-specialised workgroup (STRIDE
// threads, t = 0..STRIDE-1 among them). It walks the chunks like ReduceRing and
// takes part in nb workgroup barriers on the way, spread evenly over its steps
// and all passed by its last step: the GEMM waves run a k-loop with one barrier
// per k-tile meanwhile, and every wave of the workgroup has to reach each
// barrier. Loads in flight stay in flight across a barrier.
template <int DEPTH, typename OP, int STRIDE>
struct PacedRing {
  __device__ __forceinline__ static void run(const OP& op, int t, int total, int cpr, int64_t N,
                                             int64_t LP, int nb) {
    const int w0 = __builtin_amdgcn_readfirstlane(t & ~63);
    constexpr int per = DEPTH * STRIDE;
    // steps of this wave: whole passes of DEPTH chunks, at least one (as ReduceRing)
    const int steps = DEPTH * (total > w0 ? (total - w0 + per - 1) / per : 1);
    ChunkCursor ld, st;
    ld.init(t, total, cpr, N, LP, STRIDE);
    st = ld;
    typename OP::Chunk b[DEPTH];
#pragma unroll
    for (int i = 0; i < DEPTH - 1; ++i) {
      op.load(b[i], ld.get(), ld.lget());
      ld.advance();
    }
    int s = 0, done = 0;
    do {
#pragma unroll
      for (int i = 0; i < DEPTH; ++i) {
        op.load(b[(i + DEPTH - 1) % DEPTH], ld.get(), ld.lget());
        ld.advance();
        op.finish(b[i], st.get(), st.lget());
        st.advance();
        ++s;
        const int due = (int)((int64_t)s * nb / steps);  // nb (k-tiles) can exceed 2^25
        while (done < due) {
          __syncthreads();
          ++done;
        }
      }
    } while (s < steps);
  }
};

// Ring depth for NP peers of type PT (plus a partial if HAS_P) at OCC workgroups
// per compute unit. While a chunk is summed, DEPTH-1 chunks' loads are in
// flight; about 17 16-byte loads per wave (one chunk of 15 bfloat16 peers)
// streamed fastest on MI355X, and deeper rings were slower (more concurrent
// peer streams per wave), so small chunks get a deeper ring, within a register
// budget per lane (512 registers per SIMD lane, shared by OCC waves, minus
// addresses and the rest of the kernel); between 2 and 4.
template <int OCC, typename PT, int NP, bool HAS_P = true>
__host__ __device__ constexpr int ring_depth() {
  constexpr int loads = (HAS_P ? 2 : 0) + NP * (sizeof(PT) == 2 ? 1 : 2);  // 16-byte loads
  constexpr int regs = (HAS_P ? 8 : 0) + NP * (sizeof(PT) == 2 ? 4 : 8);   // per chunk
  constexpr int budget = OCC == 1 ? 320 : 160;
  constexpr int d_vm = 1 + (17 + loads - 1) / loads, d_reg = budget / regs;
  constexpr int d = d_vm < d_reg ? d_vm : d_reg;
  return d < 2 ? 2 : (d > 4 ? 4 : d);
}
// Whether even a depth-2 ring fits the register budget (else the generic path).
template <int OCC, typename PT, int NP>
__host__ __device__ constexpr bool ring_fits() {
  return ring_fits_regs(OCC, (int)sizeof(PT), NP);
}

// Peer counts with a compile-time ring (others take the generic path).
#define MK_RING_PEER_COUNTS(X) X(1) X(2) X(3) X(4) X(7) X(8) X(15)

// Reduce the region rows [m0, m0+rows) x cols [n0, n0+cols) of an M x N output;
// cols is a multiple of 8. All 256 threads of the workgroup take part; the
// region arguments are the same in every lane.
template <int OCC, typename PT, typename CT>
__device__ __forceinline__ void reduce_region(const float* __restrict__ P,
                                              const PT* __restrict__ peers, int n_peers,
                                              CT* __restrict__ C, int64_t M, int64_t N, int64_t m0,
                                              int64_t n0, int rows, int cols) {
  const int cpr = __builtin_amdgcn_readfirstlane(cols >> 3);
  rows = __builtin_amdgcn_readfirstlane(rows);
  const int total = rows * cpr;
  if (total <= 0) return;
  const int64_t stride = M * N;
  const int64_t base = (int64_t)__builtin_amdgcn_readfirstlane((int)m0) * N +
                       __builtin_amdgcn_readfirstlane((int)n0);
#define MK_RING(NPV)                                                                   \
  case NPV:                                                                            \
    if constexpr (ring_fits<OCC, PT, NPV>()) {                                         \
      const PT* pr[NPV];                                                               \
      _Pragma("unroll") for (int s = 0; s < NPV; ++s) pr[s] = peers + s * stride + base; \
      typedef SumOp<PT, NPV, PartialGlobal, OutC<CT>> Op;                              \
      ReduceRing<ring_depth<OCC, PT, NPV>(), Op>::run(                                 \
          Op{PartialGlobal{P + base}, pr, OutC<CT>{C + base}}, total, cpr, N, N);      \
      return;                                                                          \
    }                                                                                  \
    break;
  switch (n_peers) {
    MK_RING_PEER_COUNTS(MK_RING)
    default: break;
  }
#undef MK_RING
  auto off = [&](int q) { return base + (q / cpr) * N + (q % cpr) * 8; };
  constexpr int CH = 2;
  int q = threadIdx.x;
  for (; q + (CH - 1) * kThreads < total; q += CH * kThreads) {
    int64_t e[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) e[c] = off(q + c * kThreads);
    reduce_chunks<CH, PT, CT>(P, peers, n_peers, stride, C, e);
  }
  for (; q < total; q += kThreads) {
    int64_t e[1] = {off(q)};
    reduce_chunks<1, PT, CT>(P, peers, n_peers, stride, C, e);
  }
}

// The same for a region whose fp32 partial sits in LDS (row pitch LP elements,
// first row and column of the region at lds), by the THREADS threads of the
// workgroup (ring depths for OCC waves per SIMD). With more than 256 threads
// each lane keeps one chunk in flight: the same bytes in flight per compute
// unit as four waves at their depth, since every CU streams its tile ends at
// once (8192^3 with 7 peers, eight waves: 1080-1091 us with depth 2 against
// 1099-1105 us with depth 3). Only peer counts for which inplace_supported()
// holds.
template <int OCC, typename PT, typename CT, int THREADS = kThreads>
__device__ __forceinline__ void reduce_region_lds(const char* lds, int64_t LP,
                                                  const PT* __restrict__ peers, int n_peers,
                                                  CT* __restrict__ C, int64_t M, int64_t N,
                                                  int64_t m0, int64_t n0, int rows, int cols) {
  const int cpr = __builtin_amdgcn_readfirstlane(cols >> 3);
  rows = __builtin_amdgcn_readfirstlane(rows);
  const int total = rows * cpr;
  if (total <= 0) return;
  const int64_t stride = M * N;
  const int64_t base = (int64_t)__builtin_amdgcn_readfirstlane((int)m0) * N +
                       __builtin_amdgcn_readfirstlane((int)n0);
  const PartialLds ps{(const lds_char*)lds};
  if (n_peers == 0) {  // C = round(partial)
    typedef CopyLdsOp<CT> Op;
    ReduceRing<4, Op>::run_strided(Op{(const lds_char*)lds, OutC<CT>{C + base}}, total, cpr, N,
                                   LP, (int)threadIdx.x, THREADS);
    return;
  }
#define MK_RING(NPV)                                                                   \
  case NPV:                                                                            \
    if constexpr (ring_fits<OCC, PT, NPV>()) {                                         \
      const PT* pr[NPV];                                                               \
      _Pragma("unroll") for (int s = 0; s < NPV; ++s) pr[s] = peers + s * stride + base; \
      typedef SumOp<PT, NPV, PartialLds, OutC<CT>> Op;                                 \
      constexpr int D = THREADS > kThreads ? 2 : ring_depth<OCC, PT, NPV>();           \
      ReduceRing<D, Op>::run_strided(Op{ps, pr, OutC<CT>{C + base}}, total, cpr, N, LP,  \
                                     (int)threadIdx.x, THREADS);                       \
    }                                                                                  \
    return;
  switch (n_peers) {
    MK_RING_PEER_COUNTS(MK_RING)
    default: return;
  }
#undef MK_RING
}

// Ring depth of the streaming waves of a wave-specialised workgroup: chunks in
// flight hold only their peers' registers (the partial is read from LDS when the
// chunk is summed), within about 120 registers, between 2 and 4 chunks (a third
// chunk of 15 bfloat16 peers in flight streamed about 5% slower on MI355X: more
// concurrent peer streams per wave).
template <typename PT, int NP>
__host__ __device__ constexpr int ws_ring_depth() {
  constexpr int regs = NP * (sizeof(PT) == 2 ? 4 : 8);
  constexpr int d = 120 / regs;
  return d < 2 ? 2 : (d > 4 ? 4 : d);
}

// The same sum by the STRIDE streaming threads of a wave-specialised workgroup
// (thread t among them), taking part in nb workgroup barriers on the way
// (PacedRing). With no peers the partial is rounded and stored. Only peer counts
// for which inplace_supported(2, ...) holds: another count passes its barriers
// without touching C and returns false.
template <int STRIDE, typename PT, typename CT>
__device__ __forceinline__ bool stream_region_lds(const char* lds, int64_t LP,
                                                  const PT* __restrict__ peers, int n_peers,
                                                  CT* __restrict__ C, int64_t M, int64_t N,
                                                  int64_t m0, int64_t n0, int rows, int cols, int t,
                                                  int nb) {
  const int cpr = __builtin_amdgcn_readfirstlane(cols >> 3);
  rows = __builtin_amdgcn_readfirstlane(rows);
  const int total = rows * cpr;
  const int64_t stride = M * N;
  const int64_t base = (int64_t)__builtin_amdgcn_readfirstlane((int)m0) * N +
                       __builtin_amdgcn_readfirstlane((int)n0);
  PartialLdsLate ps;
  ps.base = (const lds_char*)lds;
  if (total > 0) {
    if (n_peers == 0) {
      typedef CopyLdsOp<CT> Op;
      PacedRing<4, Op, STRIDE>::run(Op{(const lds_char*)lds, OutC<CT>{C + base}}, t, total, cpr,
                                    N, LP, nb);
      return true;
    }
#define MK_RING(NPV)                                                                     \
  case NPV:                                                                              \
    if constexpr (ring_fits<2, PT, NPV>()) {                                             \
      const PT* pr[NPV];                                                                 \
      _Pragma("unroll") for (int s = 0; s < NPV; ++s) pr[s] = peers + s * stride + base;   \
      typedef SumOp<PT, NPV, PartialLdsLate, OutC<CT>> Op;                               \
      PacedRing<ws_ring_depth<PT, NPV>(), Op, STRIDE>::run(Op{ps, pr, OutC<CT>{C + base}}, t,  \
                                                           total, cpr, N, LP, nb);       \
      return true;                                                                       \
    }                                                                                    \
    break;
    switch (n_peers) {
      MK_RING_PEER_COUNTS(MK_RING)
      default: break;
    }
#undef MK_RING
  }
  for (int i = 0; i < nb; ++i) __syncthreads();
  return total <= 0;
}

// Rounds the fp32 partial of a region in LDS (row pitch LP) to OT and stores it
// to rows [m0, m0+rows) x cols [n0, n0+cols) of an N-column output.
template <typename OT>
__device__ __forceinline__ void copy_region_lds(const char* lds, int64_t LP, OT* __restrict__ out,
                                                int64_t N, int64_t m0, int64_t n0, int rows,
                                                int cols) {
  const int cpr = __builtin_amdgcn_readfirstlane(cols >> 3);
  rows = __builtin_amdgcn_readfirstlane(rows);
  const int total = rows * cpr;
  if (total <= 0) return;
  const int64_t base = (int64_t)__builtin_amdgcn_readfirstlane((int)m0) * N +
                       __builtin_amdgcn_readfirstlane((int)n0);
  typedef CopyLdsOp<OT> Op;
  ReduceRing<4, Op>::run(Op{(const lds_char*)lds, OutC<OT>{out + base}}, total, cpr, N, LP);
}

// A reduce unit in two phases, for a reducer that takes the unit before its
// tile's partial is published. Phase 1 sums the region's peers into LDS (row
// pitch LP); it reads nothing the GEMM produces. Phase 2, once the partial is
// published, adds it and writes C. Together they make the same float32
// additions as reduce_region. Only peer counts for which inplace_supported()
// holds.
template <int OCC, typename PT>
__device__ __forceinline__ void reduce_region_peers_lds(char* lds, int64_t LP,
                                                        const PT* __restrict__ peers, int n_peers,
                                                        int64_t M, int64_t N, int64_t m0,
                                                        int64_t n0, int rows, int cols) {
  const int cpr = __builtin_amdgcn_readfirstlane(cols >> 3);
  rows = __builtin_amdgcn_readfirstlane(rows);
  const int total = rows * cpr;
  if (total <= 0) return;
  const int64_t stride = M * N;
  const int64_t base = (int64_t)__builtin_amdgcn_readfirstlane((int)m0) * N +
                       __builtin_amdgcn_readfirstlane((int)n0);
  const OutLds out{(lds_char*)lds};
#define MK_RING(NPV)                                                                    \
  case NPV:                                                                             \
    if constexpr (ring_fits<OCC, PT, NPV>()) {                                          \
      const PT* pr[NPV];                                                                \
      _Pragma("unroll") for (int s = 0; s < NPV; ++s) pr[s] = peers + s * stride + base;  \
      typedef SumOp<PT, NPV, NoPartial, OutLds> Op;                                     \
      ReduceRing<ring_depth<OCC, PT, NPV, false>(), Op>::run(Op{NoPartial{}, pr, out},   \
                                                             total, cpr, N, LP);        \
    }                                                                                   \
    return;
  switch (n_peers) {
    MK_RING_PEER_COUNTS(MK_RING)
    default: return;
  }
#undef MK_RING
}
template <typename CT>
__device__ __forceinline__ void reduce_region_finish(const float* __restrict__ P,
                                                     const char* lds, int64_t LP,
                                                     CT* __restrict__ C, int64_t N, int64_t m0,
                                                     int64_t n0, int rows, int cols) {
  const int cpr = __builtin_amdgcn_readfirstlane(cols >> 3);
  rows = __builtin_amdgcn_readfirstlane(rows);
  const int total = rows * cpr;
  if (total <= 0) return;
  const int64_t base = (int64_t)__builtin_amdgcn_readfirstlane((int)m0) * N +
                       __builtin_amdgcn_readfirstlane((int)n0);
  typedef PresumOp<CT> Op;
  ReduceRing<4, Op>::run(Op{PartialGlobal{P + base}, (const lds_char*)lds, OutC<CT>{C + base}},
                         total, cpr, N, LP);
}

// Phase 2 for a tile computed in NP k-parts (partials NP * M * N floats apart,
// same layout): C = round(peer sum + ((P_0 + P_1) + ...)).
template <int NP, typename CT>
__device__ __forceinline__ void reduce_region_finish_parts(const float* __restrict__ P,
                                                           int64_t part_stride, const char* lds,
                                                           int64_t LP, CT* __restrict__ C,
                                                           int64_t N, int64_t m0, int64_t n0,
                                                           int rows, int cols) {
  const int cpr = __builtin_amdgcn_readfirstlane(cols >> 3);
  rows = __builtin_amdgcn_readfirstlane(rows);
  const int total = rows * cpr;
  if (total <= 0) return;
  const int64_t base = (int64_t)__builtin_amdgcn_readfirstlane((int)m0) * N +
                       __builtin_amdgcn_readfirstlane((int)n0);
  typedef PresumOp<CT, PartialGlobalN<NP>> Op;
  ReduceRing<4, Op>::run(Op{PartialGlobalN<NP>{P + base, (uint32_t)(part_stride * 4)},
                            (const lds_char*)lds, OutC<CT>{C + base}},
                         total, cpr, N, LP);
}

}  // namespace mk
