// mk_kernels.h -- interface between the host library (mk_api.cpp) and the
// kernels (mk_kernels.hip). Internal; the public ABI is include/mk.h.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk.h"

namespace mk {

// Workspace control words, each on its own 128-byte line (kSlotWords 64-bit
// words). Counters that every tile updates are kept per XCD: one address hit by
// all 256 workgroups serialises their atomics (about 2.9 us per operation
// measured on MI355X, against 0.35 us for an XCD's own line).
// Per-XCD words, at S_XCD_BASE + kXcdWords * xcd + word.
enum XcdSlot : int {
  X_COMPUTE_NEXT = 0,  // next tile of the XCD's queue to compute
  X_REDUCE_NEXT,       // next reduce unit of the XCD's queue
  X_ARRIVE,            // workgroups that arrived on the XCD (their rank)
  X_COMPUTED,          // tiles published
  X_REDUCED,           // reduce units (tile row slabs) done
  X_BUSY_C,            // summed compute-tile ticks
  X_BUSY_R,            // summed reduce-unit ticks (flag waits excluded)
  X_WAIT_R,            // summed flag-wait ticks
  X_SWITCHES,          // workgroup role changes
  X_RBC,               // reduce units done by workgroups that prefer compute (draining)
  X_CBR,               // tiles computed by workgroups that prefer reducing (helping)
  X_INPLACE,           // tiles reduced in place by the workgroup that computed them
  X_PHYS,              // 1 + the hardware XCD id of the workgroups serving this queue (0 = none yet)
  X_STREAM,            // workgroups streaming a reduce now (in place or a handed-over unit)
  X_PUB,               // dynamic hand-over: tiles of the queue published for reducers
  X_PUB_T,             // summed ticks from a partial's store-complete wait to its flag store
  X_ACQ_T,             // summed ticks from a flag seen set to the end of its acquire
  X_NPUB,              // tiles published through a flag
  X_NACQ,              // reduce units that acquired a flag
  kXcdWords
};
constexpr int kMaxXcd = 16;
enum Slot : int {
  S_EXIT = 0,          // workgroups that have left the persistent loop
  S_ERROR,             // device error word (mk_status_t), kept across calls
  S_ABORT,             // set on error: every workgroup leaves its loop
  S_LOCK,              // controller try-lock
  S_TARGET,            // (epoch << 32) | reducer target published by the controller
  S_UPDATES,           // controller target changes
  S_NTRACE,            // controller trace entries written
  S_TSTART,            // min start tick
  S_TEND,              // max exit tick
  S_PING,              // flag hand-off microbenchmark: (call << 32) | step, one per side
  S_PONG,
  S_PAYLOAD,           // ... and the data word each hand-off carries
  S_XCD_BASE,          // per-XCD words follow
  S_COUNT = S_XCD_BASE + kXcdWords * kMaxXcd
};

constexpr int kSlotWords = 16;
constexpr int kThreadsHost = 256;  // workgroup size of every kernel

// Fixed device-memory workspace of the allocation-free entry point, one per GPU:
// control words, then tile flags, then fp32 partials (sizes in mk.h).
constexpr size_t kScratchSlotBytes = ((size_t)S_COUNT * kSlotWords * 8 + 255) / 256 * 256;
constexpr size_t kScratchFlags = MK_NOALLOC_MAX_TILE_FLAGS;
constexpr size_t kScratchPartialBytes = MK_NOALLOC_PARTIAL_BYTES;
constexpr size_t kScratchBytes = kScratchSlotBytes + kScratchFlags * 4 + kScratchPartialBytes;

// SHAPE_WS, SHAPE_WS128: 64x256 or 128x128 tiles in the wave-specialised kernel
// (384 or 512 threads, the GEMM of one tile overlapping the reduce of the one
// before, every tile in place)
enum TileShape : int {
  SHAPE_AUTO = 0, SHAPE_256 = 1, SHAPE_128 = 2, SHAPE_64 = 3, SHAPE_WS = 4, SHAPE_WS128 = 5
};
constexpr int kShapes = 6;
constexpr bool is_ws(int shape) { return shape == SHAPE_WS || shape == SHAPE_WS128; }

// Tile queues and flag protocol of a persistent launch of G workgroups on a
// device with `cus` compute units. gfx950 groups 32 compute units per XCD, each
// XCD with its own L2; a kernel takes its queue from the hardware XCD id modulo
// n_xcd. The XCD-local flag protocol (scope 0: stores complete, relaxed flag,
// no L2 write-back) is valid only while every queue is served by workgroups of
// one XCD: the device then has cus/32 XCDs and the grid, dealt to the XCDs in
// turn, is a multiple of that count. Otherwise every tile goes through one
// queue with agent-scope release and acquire (scope 1), which is correct across
// XCDs. scope_opt is the requested scope (MK_OPT_FLAG_SCOPE).
inline void queue_plan(int cus, int G, int scope_opt, int& n_xcd, int& scope) {
  const int n = cus > 0 && cus % 32 == 0 ? cus / 32 : 0;
  const bool per_xcd = n >= 1 && n <= kMaxXcd && G > 0 && G % n == 0;
  n_xcd = per_xcd ? n : 1;
  scope = per_xcd ? (scope_opt != 0 ? 1 : 0) : 1;
}

// Peer counts that have a compile-time reduce ring (0: the partial rounded and
// stored), and whether that ring fits the register budget of a lane at `occ`
// workgroups per compute unit (peers of peer_bytes bytes: 8 registers of
// partial plus 4 or 8 per peer per chunk, two chunks at least). A tile can be
// reduced in place (partial in LDS) only then. Shared by the host (which counts
// the tiles handed to reducers) and the kernels.
constexpr bool ring_peer_count(int np) {
  return np == 0 || np == 1 || np == 2 || np == 3 || np == 4 || np == 7 || np == 8 || np == 15;
}
constexpr bool ring_fits_regs(int occ, int peer_bytes, int np) {
  return 2 * (8 + np * (peer_bytes == 2 ? 4 : 8)) <= (occ == 1 ? 320 : 160);
}
constexpr bool inplace_supported(int occ, int peer_bytes, int np) {
  return ring_peer_count(np) && ring_fits_regs(occ, peer_bytes, np);
}
// Tiles of XCD x's queue (T tiles over n_xcd XCDs) and how many of them are
// reduced in place (the last ones).
constexpr int xcd_tiles(int T, int n_xcd, int x) {
  return (int)(((int64_t)(x + 1) * T) / n_xcd - ((int64_t)x * T) / n_xcd);
}
constexpr int xcd_inplace(int cnt, int n_inplace, bool supported) {
  if (!supported) return 0;
  return n_inplace < cnt ? (n_inplace > 0 ? n_inplace : 0) : cnt;
}

struct FusedArgs {
  const uint16_t* A;
  const uint16_t* B;
  const void* peers;
  void* C;
  float* P;                    // fp32 partial tiles, [M][N]
  int* flags;                  // one per tile, holds the epoch of the call that published it
  unsigned long long* pub;     // dynamic hand-over: slot q0 + s of XCD x's queue holds
                               // (epoch << 32) | tile of the s-th tile it published
  unsigned long long* slots;   // S_COUNT * kSlotWords words
  mk_telemetry_t* tel;         // optional
  int64_t M, N, K;
  int n_peers, tiles_m, tiles_n, T;
  int G;                       // workgroups in the grid
  int epoch;                   // this call's flag value (never 0)
  int init_target;             // reducer target before the controller's first update
  int adaptive;                // controller on/off
  float seed_x;                // controller seed share
  int ctrl_period;
  int withhold_tile;           // debug: -1 = off
  int n_xcd;                   // XCDs of the device; tiles are queued per XCD
  int flag_scope;              // 0: producer and consumer share an XCD's L2; 1: agent scope
  int shared_lines;            // 1: a 128-byte line of the partial can hold two reduce units'
                               // rows (N not a multiple of 32): consumers acquire at agent
                               // scope; 0: every line belongs to one unit, no invalidate
  int reducer_cap;             // controller's upper bound on reducers while compute remains
  int n_inplace;               // per XCD: last tiles of the queue reduced in place
  int T_r;                     // tiles handed to reducers (T minus the in-place ones)
  int early;                   // 1: a reducer may take a unit whose tile is still being
                               // computed, and sums its peers while it waits
  int one_tile;                // 1: every tile reduced in place and one workgroup per tile: the
                               // tile is the workgroup's index, no claim or counter is used
  int dyn;                     // 1: each tile is reduced in place or handed over when its GEMM
                               // ends, by the streaming slots free at that moment (the
                               // controller's target counts streaming workgroups); 0: the
                               // last n_inplace tiles of each queue are in place
  int ksplit;                  // 1, or 2 (early reduce only): a tile is computed as two
                               // k-halves, each its own compute item, partial slice
                               // (P + half*M*N) and flag (flags[2*tile + half])
  // GEMM+ReduceScatter share (rs = 1): rows [own0, own1) are reduced into C
  // ([own1-own0, N]) with peers [n_peers, own1-own0, N]; the partial of every
  // other row is rounded to the peer type and stored to send ([M, N]). Tiles
  // in tile rows [tmo0, tmo1) are handed over, the others published in place.
  int rs;
  int tmo0, tmo1;              // tile rows that hold owned rows: [tmo0, tmo1)
  int64_t own0, own1;
  void* send;
  unsigned long long spin_limit;  // flag-wait limit in 100 MHz ticks
  int static_tiles;            // 1: every tile reduced in place, tiles dealt to the workgroups
                               // in a fixed order (inplace_kernel): no claim, flag or counter
  int ws_wide;                 // wave-specialised 128x128 tiles: 1 = four streaming waves
  int waves8;                  // in-place kernel (static_tiles, 256x256): eight waves
};

struct GemmArgs {
  const uint16_t* A;
  const uint16_t* B;
  float* P;
  int64_t M, N, K;
  int tiles_m, tiles_n;
  int n_xcd;  // workgroup b runs on XCD b % n_xcd; 1 = no XCD-aware mapping
  int waves8;  // 256x256 tiles: eight waves per workgroup (512 threads), else four
};

struct ReduceArgs {
  const float* P;      // rows [0, M) of the region
  const void* peers;   // peer p's region at peers + p * peer_stride elements
  void* C;
  int64_t M, N;        // region rows and columns (dense, row pitch N)
  int64_t peer_stride; // elements between two peers' arrays
  int n_peers;
  int pad_;
};

// AllGather+GEMM share: this GPU's row shard of the activations, the other
// GPUs' shards (standing in for data they broadcast), the gathered matrix and
// C = gathered x B. The gathered matrix is landed in bands of BM rows, each cut
// into at most kAgMaxPieces column pieces of KP columns (a multiple of the GEMM's
// k-tile); one flag per (band, piece) says the piece has landed.
constexpr int kAgMaxPieces = 32;
struct AgArgs {
  const uint16_t* A_local;     // [Ms, K], rank `rank`'s shard
  const uint16_t* peers;       // [P-1, Ms, K], the other shards in rank order (rank left out)
  uint16_t* A_full;            // [P*Ms, K], shard q at rows [q*Ms, (q+1)*Ms)
  const uint16_t* B;           // [K, N]
  void* C;                     // [P*Ms, N]
  int* landed;                 // [NB][kAgMaxPieces]: 1 once the piece has landed (zero between calls)
  unsigned long long* slots;   // S_COUNT * kSlotWords words
  int64_t M, N, K, Ms;         // M = P*Ms
  int64_t KP;                  // columns per piece
  int P, rank;
  int bps;                     // bands per shard (Ms / BM)
  int NB;                      // bands (M / BM)
  int npc;                     // pieces per band (ceil(K / KP))
  int ktpp;                    // k-tiles per piece (KP / BK)
  int inloop;                  // 1: a tile waits for each piece in its k-loop; 0: for every
                               // piece of its band before the GEMM (pieces share cache lines)
  int tiles_n, T;
  int G, n_xcd;
  int n_comm;                  // workgroups that only land pieces while any are left
  int flag_scope;              // 0: pieces landed and read behind one XCD's L2; 1: agent scope
  unsigned long long spin_limit;  // piece-wait limit in 100 MHz ticks
};

// Baseline of the AllGather+GEMM share: the gathered matrix by a copy kernel,
// then this GEMM kernel (one workgroup per tile) writing C in its type.
struct AgCopyArgs {
  const uint16_t* A_local;
  const uint16_t* peers;
  uint16_t* A_full;
  int64_t Ms, K;
  int P, rank;
};

// variant: the dynamic hand-over kernel (256x256 and 128x128 tiles), or four
// streaming waves instead of two (wave-specialised 128x128 tiles)
const void* fused_kernel_ptr(int shape, int pt, int ct, int variant);
const void* ag_kernel_ptr(int shape, int ct);
const void* gemm_kernel_ptr(int shape, int waves8);
const void* reduce_kernel_ptr(int pt, int ct);
int shape_bm(int shape);
int shape_threads(int shape, int variant);  // workgroup size of the fused kernel of a shape
// Whether a wave-specialised call with 128x128 tiles streams with four waves:
// when each streaming lane holds one chunk in flight while it sums another (the
// ring depth of its peer count, 120 registers over the chunk's, is at most 2).
constexpr bool ws_wide(int shape, int peer_bytes, int n_peers) {
  return shape == SHAPE_WS128 && n_peers > 0 && 120 / (n_peers * (peer_bytes == 2 ? 4 : 8)) <= 2;
}
int shape_bn(int shape);

hipError_t launch_ws_init(int* flags, int n_flags, unsigned long long* slots, hipStream_t s);
// Device address of the allocation-free workspace on the current device (looked
// up from its symbol; the caller keeps it per device).
hipError_t noalloc_scratch_address(void** p);
hipError_t launch_clear_error(unsigned long long* slots, hipStream_t s);
hipError_t launch_fused(int shape, int pt, int ct, const FusedArgs& a, hipStream_t s);
hipError_t launch_gemm(int shape, const GemmArgs& a, hipStream_t s);
hipError_t launch_reduce(int pt, int ct, const ReduceArgs& a, int grid, hipStream_t s);
hipError_t launch_ag(int shape, int ct, const AgArgs& a, hipStream_t s);
hipError_t launch_pingpong(unsigned long long* slots, unsigned call, int iters, int scope,
                           int cross_xcd, unsigned long long limit, unsigned long long* out,
                           hipStream_t s);
hipError_t launch_ag_copy(const AgCopyArgs& a, int grid, hipStream_t s);
hipError_t launch_gemm_c(int shape, int ct, const GemmArgs& a, void* C, hipStream_t s);
hipError_t launch_mfma_peak(int iters, int grid, float* out, hipStream_t s);

}  // namespace mk
