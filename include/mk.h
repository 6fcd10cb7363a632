/*
 * mk.h -- C ABI of libmk.so: one GPU's share of a tile-granular fused
 * GEMM+AllReduce on AMD Instinct MI355X (gfx950).
 *
 * The operation is the "GEMM + AllReduce (TP)" kernel of "mKernel: Fast
 * Multi-GPU, Multi-Node Fused Kernels" (arXiv 2609.13585), thelatestinai.com
 * page, Table 3: a compute -> communication kernel whose output tiles are
 * reduced across the GPUs of a tensor-parallel group. With K split across P
 * GPUs, the share computed here is
 *
 *     C[i,j] = sum_{k<K} A[i,k] * B[k,j]  +  sum_{p<P-1} peers[p][i,j]
 *
 * where peers[] stands for the P-1 partial products that the other GPUs would
 * deliver (here: inputs already resident in device memory).
 *
 * The fused entry point runs one persistent kernel whose workgroups take one
 * of two roles (same page, Figure 2, items 1 and 6, and the abstract):
 *   - compute workgroups run the bf16 matrix-core GEMM of a tile, store its
 *     fp32 partial to a library workspace and set that tile's readiness flag;
 *   - reducer workgroups wait for a tile's flag, then add the peer partials and
 *     write C.
 * An on-GPU controller (Figure 2 caption, Figure 7) reads progress counters and
 * publishes how many workgroups should be reducers. Tiles can instead be
 * reduced in place by the workgroup that computed them, through its LDS, with
 * no partial in memory and no flag (MK_OPT_INPLACE): on MI355X that is the
 * faster path for most tiles, and by default only the first tiles of each
 * XCD's queue of a memory-bound shape are handed to reducers.
 *
 * The same library holds the shares of two more kernels of that Table 3
 * (GEMM + ReduceScatter, AllGather + GEMM: mk_gemm_rs_local, mk_gemm_ag_local),
 * the two-kernel and two-stream comparison schedules, and a flag hand-off
 * microbenchmark.
 *
 * Layout of every tensor argument: dense, row-major, 16-byte aligned device
 * memory owned by the caller:
 *   A      [M, K]            bfloat16
 *   B      [K, N]            bfloat16
 *   peers  [n_peers, M, N]   peer_dtype (bfloat16 or float32), one contiguous block
 *   C      [M, N]            c_dtype    (bfloat16 or float32)
 * Accumulation is float32. The peer partials are summed in index order
 * (peers[0] + peers[1] + ...), then the local fp32 partial is added; the sum is
 * rounded once to c_dtype, round to nearest even (with no peers, C is the
 * rounded partial). The result is bitwise identical for every reducer count,
 * every option below, the adaptive controller and the two-kernel baseline,
 * except where a tile is computed as two k-halves (MK_OPT_KSPLIT, automatic for
 * few-tile shapes): its local partial is then the float32 sum of the halves'
 * partials, which can differ from one k-loop in the last bit.
 *
 * Supported shapes: M >= 0 (any), N and K multiples of 8 (16-byte rows),
 * N <= 4194304 (2^22).
 * M == 0 or N == 0 is a no-op. K == 0 gives C = sum of peers. n_peers == 0
 * gives C = A*B. 0 <= n_peers <= MK_MAX_PEERS.
 *
 * Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 * stream). No host<->device copy happens inside a call. The library keeps one
 * workspace per (device, stream): the fp32 partial buffer, tile flags and
 * counters. It is created on first use, grows as needed and lives until
 * process exit or mk_workspace_reset(). Calls on one stream are ordered by the
 * stream; calls on different streams use different workspaces.
 *
 * Errors: every function returns an mk_status_t. Argument validation never
 * dereferences device pointers, so it runs without touching the GPU. Errors
 * raised on the device (a reducer wait that exceeded its time limit) are
 * reported by mk_stream_status(). mk_last_error() gives a thread-local text.
 * Every device-side wait is bounded (MK_OPT_SPIN_TIMEOUT_US), so a stuck
 * hand-off ends the kernel with MK_ERR_TIMEOUT rather than hanging it.
 */
#ifndef MK_H_
#define MK_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MK_OK = 0,
  MK_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad dtype, negative size, aliasing */
  MK_ERR_UNSUPPORTED = 2, /* valid but outside the supported envelope (N or K not %8) */
  MK_ERR_HIP = 3,         /* a HIP runtime call failed; see mk_last_error() */
  MK_ERR_TIMEOUT = 4,     /* a device-side wait (tile flag, landed piece) passed its limit */
  MK_ERR_NO_DEVICE = 5,   /* no usable gfx950 device */
  MK_ERR_WORKSPACE = 6,   /* workspace allocation failed */
  MK_ERR_INTERNAL = 7     /* a persistent kernel ended with work left undone */
} mk_status_t;

typedef enum { MK_DT_BF16 = 0, MK_DT_F32 = 1 } mk_dtype_t;

/* n_reduce_wg value that hands the reducer count to the on-GPU controller. */
#define MK_ADAPTIVE (-1)
#define MK_MAX_PEERS 64
/* Most chunks of mk_gemm_ar_two_stream. */
#define MK_MAX_CHUNKS 64
/* Limits of mk_gemm_ar_local_noalloc's fixed workspace (per GPU). */
#define MK_NOALLOC_PARTIAL_BYTES (32u << 20) /* fp32 partials of tiles handed to reducers */
#define MK_NOALLOC_MAX_TILE_FLAGS 65536      /* tiles times k-parts per tile */

/* Telemetry written by the fused kernel when the caller passes a device buffer
 * of sizeof(mk_telemetry_t) bytes (else NULL). Times are in ticks of the GPU's
 * constant 100 MHz clock. The controller trace holds one entry per controller
 * update (Figure 7 of the thelatestinai.com page plots the same quantity). */
#define MK_TRACE_CAP 512
typedef struct {
  uint64_t t;         /* tick of the update */
  int32_t computed;   /* tiles whose partial was published */
  int32_t reduced;    /* tiles whose C was written */
  int32_t target;     /* published reducer target */
  int32_t spare;      /* workgroups streaming a reduce at the update (dynamic hand-over) */
} mk_trace_entry_t;

typedef struct {
  uint64_t t_start;          /* first workgroup start */
  uint64_t t_end;            /* last workgroup exit */
  uint64_t busy_compute;     /* sum over compute tiles of their duration */
  uint64_t busy_reduce;      /* sum over reduce tiles, excluding flag waits */
  uint64_t wait_reduce;      /* sum of reducer flag waits */
  int32_t tiles;             /* tile count of the call */
  int32_t grid;              /* workgroups launched */
  int32_t initial_target;
  int32_t final_target;
  int32_t n_updates;         /* controller updates that changed the target */
  int32_t n_trace;           /* valid entries in trace[] (<= MK_TRACE_CAP) */
  int32_t role_switches;     /* workgroup role changes, summed */
  int32_t reduced_by_compute;/* tiles reduced by compute-role workgroups (draining) */
  int32_t computed_by_reducers; /* tiles computed by reducer-role workgroups with nothing to reduce */
  int32_t n_xcd;             /* XCDs; each XCD computes and reduces its own share of tiles */
  /* Tile-flag overhead (the two halves of a hand-over that Table 2's caption of the
   * thelatestinai.com page separates: a write completing, then becoming visible):
   * publish_ticks sums, over the tiles handed to reducers, the ticks from the
   * computing workgroup's wait for its partial stores to complete to its flag
   * store; acquire_ticks sums, over reduce units, the ticks from the poll that
   * sees the flag to the end of the acquire (wait_reduce, which also counts the
   * time spent waiting for the tile to be computed, includes it). */
  uint64_t publish_ticks;
  uint64_t acquire_ticks;
  int32_t published;         /* tiles handed over through a flag */
  int32_t acquired;          /* reduce units that acquired a flag */
  mk_trace_entry_t trace[MK_TRACE_CAP];
} mk_telemetry_t;

/*
 * mk_gemm_ar_local -- fused persistent kernel (one launch).
 *   A, B, peers, C : device pointers, layout above. peers may be NULL iff
 *                    n_peers == 0. C must not overlap A, B or peers.
 *   n_peers        : P-1, the number of peer partials.
 *   M, N, K        : K is this GPU's K-shard length.
 *   peer_dtype     : MK_DT_BF16 or MK_DT_F32.
 *   c_dtype        : MK_DT_BF16 or MK_DT_F32.
 *   stream         : hipStream_t (NULL = default stream).
 *   n_reduce_wg    : 0 .. G-1 dedicated reducer workgroups (G =
 *                    mk_fused_grid() of these arguments), or MK_ADAPTIVE. With 0, compute
 *                    workgroups reduce the tiles once no GEMM tile is left;
 *                    the same draining applies in every mode. MK_ADAPTIVE also
 *                    lets the library take the wave-specialised schedule
 *                    (MK_OPT_TILE_SHAPE); forced by that option, it ignores
 *                    n_reduce_wg (it has no reducer workgroups: each workgroup
 *                    reduces its own tiles with two of its waves).
 *   telemetry      : NULL or a device buffer of sizeof(mk_telemetry_t); a call with
 *                    telemetry never takes the wave-specialised schedule.
 * Returns MK_OK once the kernel is enqueued.
 */
mk_status_t mk_gemm_ar_local(const void* A, const void* B, const void* peers, int n_peers,
                             void* C, int64_t M, int64_t N, int64_t K, int peer_dtype,
                             int c_dtype, void* stream, int n_reduce_wg, void* telemetry);

/*
 * mk_gemm_ar_local_noalloc -- mk_gemm_ar_local for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. Same arguments, kernels and result as mk_gemm_ar_local
 * (bitwise, with the same exception for tiles computed as two k-halves); it calls
 * no hipMalloc, hipFree or allocating library routine and no hipMemsetAsync.
 * Its workspace is a fixed array in device memory, one per GPU the library runs
 * on, held until the process ends: control words, MK_NOALLOC_MAX_TILE_FLAGS tile
 * flags and MK_NOALLOC_PARTIAL_BYTES of fp32 partials. The first call on a
 * device (and the first after mk_workspace_reset) clears its flags and control
 * words with a fill kernel on `stream`.
 *   - A call whose default schedule would hand tiles to reducers with more
 *     partial bytes than that (M * N * 4 per k-part) reduces every tile in place
 *     instead (same bits); for peer counts that cannot be reduced in place (those
 *     outside 0-4, 7, 8, 15, or fp32 peers beyond what fits a lane's registers)
 *     it returns MK_ERR_UNSUPPORTED, as it does for more tiles times k-parts
 *     than there are flags. Nothing is launched then.
 *   - Every call on one GPU shares that GPU's workspace. Calls that overlap on
 *     one GPU (on two streams, or from two threads without ordering) race and
 *     give undefined results; calls ordered on one stream are safe.
 *   - Device-side errors are reported by mk_stream_status on the call's stream.
 */
mk_status_t mk_gemm_ar_local_noalloc(const void* A, const void* B, const void* peers,
                                     int n_peers, void* C, int64_t M, int64_t N, int64_t K,
                                     int peer_dtype, int c_dtype, void* stream, int n_reduce_wg,
                                     void* telemetry);

/*
 * mk_gemm_then_reduce_baseline -- the unfused schedule of Figure 1 on the
 * thelatestinai.com page: a GEMM kernel that writes every fp32 partial tile,
 * then a separate reduce kernel, in order on `stream`. Same arguments and
 * result as mk_gemm_ar_local (bitwise).
 */
mk_status_t mk_gemm_then_reduce_baseline(const void* A, const void* B, const void* peers,
                                         int n_peers, void* C, int64_t M, int64_t N, int64_t K,
                                         int peer_dtype, int c_dtype, void* stream);

/*
 * mk_gemm_ar_two_stream -- the stream-overlap schedule of Figure 1(b) on the
 * thelatestinai.com page: the output rows are cut into n_chunks chunks of
 * whole tile rows; the GEMM kernel of each chunk runs on `stream`, and the
 * reduce kernel of a chunk runs on a second stream of the library as soon as
 * that chunk's GEMM kernel has ended (an event), overlapping the GEMM of the
 * following chunks. Kernel boundaries are the only readiness signal; no flag
 * is involved. The second stream (default priority) and its events belong to
 * the (device, stream) workspace. The call is ordered on `stream` like the
 * others: every reduce waits for an event recorded on `stream` after its
 * chunk's GEMM, and `stream` waits for the last reduce.
 * With MK_OPT_STREAM_CU_SPLIT = R > 0 the two streams partition the chip
 * instead of sharing it (AMD CU-masked streams, the static counterpart of the
 * role split): the GEMM kernels run on a library stream masked to all but R
 * compute units and the reduce kernels on one masked to the other R; the GEMM
 * stream first waits for an event recorded on `stream`.
 *   n_chunks : 0 = automatic (4), else 1..MK_MAX_CHUNKS; at most the number of
 *              tile rows (the tile shape is chosen as for the fused kernel).
 * Other arguments and result as mk_gemm_ar_local (bitwise: the same GEMM tile
 * and reduce code, the same sum order).
 */
mk_status_t mk_gemm_ar_two_stream(const void* A, const void* B, const void* peers, int n_peers,
                                  void* C, int64_t M, int64_t N, int64_t K, int peer_dtype,
                                  int c_dtype, void* stream, int n_chunks);

/*
 * mk_gemm_rs_local -- one GPU's share of the "GEMM + ReduceScatter (TP)" kernel
 * of Table 3 on the thelatestinai.com page (compute -> communication: each
 * output tile is added into the buffer of the GPU that owns it). This GPU owns
 * output rows [own_m0, own_m1) (own = own_m1 - own_m0 rows). With its local
 * partial Pl = A*B (fp32 accumulation):
 *   C[i - own_m0, j] = round_c((peers[0][i-own_m0][j] + ... + peers[n-1][..][j]) + Pl[i][j])
 *                                                    for own_m0 <= i < own_m1,
 *   send[i, j]       = round_peer(Pl[i][j])          for every other row i,
 * i.e. the owned slice is reduced here (same sum order as mk_gemm_ar_local) and
 * every other row is published, rounded to the peer type, for its owner (which
 * receives it as one of its peer partials).
 *   A [M, K] bf16; B [K, N] bf16;
 *   peers [n_peers, own, N] peer_dtype: the other GPUs' partials of the owned rows;
 *   C [own, N] c_dtype; send [M, N] peer_dtype, rows of [own_m0, own_m1) left
 *   untouched (send may be NULL when every row is owned).
 * One persistent launch of the fused kernel. The tile rows that hold owned rows
 * lead every XCD's queue and are handed to reducers through the workspace and
 * tile flags (64-row units: owned rows reduced, the others published); every
 * other tile is rounded and published by the workgroup that computed it, in
 * place. n_reduce_wg: 0 .. G-1 dedicated reducers (G as mk_fused_grid() with
 * MK_OPT_EARLY off) or MK_ADAPTIVE. Any n_peers <= MK_MAX_PEERS. Same alignment
 * and overlap rules as above; C and send must not overlap each other or any
 * input.
 */
mk_status_t mk_gemm_rs_local(const void* A, const void* B, const void* peers, int n_peers, void* C,
                             void* send, int64_t M, int64_t N, int64_t K, int64_t own_m0,
                             int64_t own_m1, int peer_dtype, int c_dtype, void* stream,
                             int n_reduce_wg);

/* mk_gemm_rs_baseline -- the same result (bitwise) unfused: the GEMM kernel
 * writes the fp32 partial of all M rows, then the reduce kernel sums the owned
 * rows and rounds the other rows to the peer type. Any n_peers <= MK_MAX_PEERS. */
mk_status_t mk_gemm_rs_baseline(const void* A, const void* B, const void* peers, int n_peers,
                                void* C, void* send, int64_t M, int64_t N, int64_t K,
                                int64_t own_m0, int64_t own_m1, int peer_dtype, int c_dtype,
                                void* stream);

/*
 * mk_gemm_ag_local -- one GPU's share of the "AllGather + GEMM (TP)" kernel of
 * Table 3 on the thelatestinai.com page (communication -> compute: each GPU's
 * row shard of the activations is broadcast to every GPU, and the GEMM consumes
 * gathered rows in row chunks as they arrive). With P = n_peers + 1 GPUs, this
 * one of rank `rank`:
 *   A_full[q*Ms + i, k] = (q == rank ? A_local : peers_A[q < rank ? q : q-1])[i, k]
 *   C[i, j]             = round_c( sum_k A_full[i, k] * B[k, j] )   (fp32 accumulation)
 *   A_local [Ms, K] bf16: this GPU's shard;
 *   peers_A [n_peers, Ms, K] bf16: the other GPUs' shards in rank order, `rank`
 *           left out (inputs standing in for the broadcast data);
 *   A_full  [P*Ms, K] bf16: the gathered matrix (written);
 *   B [K, N] bf16; C [P*Ms, N] c_dtype (written).
 * One persistent launch. The other GPUs' shards are landed in A_full in bands of
 * tile rows (128 or 256), each in pieces with a counter per band; a tile is
 * computed once its band has landed, this GPU's own bands at once (read from
 * A_local). A workgroup whose band is missing lands pieces itself, so any
 * n_comm_wg is deadlock-free. n_comm_wg: workgroups that prefer landing,
 * 0 .. mk_ag_grid()-1, or MK_ADAPTIVE for the library's default. Requires Ms a
 * multiple of 128, N and K multiples of 8, 16-byte aligned pointers, rank in
 * [0, n_peers], n_peers <= MK_MAX_PEERS; else MK_ERR_INVALID_ARG or
 * MK_ERR_UNSUPPORTED. A_full and C must not overlap each other or any input.
 * Asynchronous on `stream`; a band wait past MK_OPT_SPIN_TIMEOUT_US stops the
 * kernel and sets the error word that mk_stream_status returns.
 */
mk_status_t mk_gemm_ag_local(const void* A_local, const void* peers_A, int n_peers, void* A_full,
                             const void* B, void* C, int64_t Ms, int64_t N, int64_t K, int rank,
                             int c_dtype, void* stream, int n_comm_wg);

/* mk_gemm_ag_baseline -- the same result (bitwise) unfused: a copy kernel
 * gathers every shard into A_full, then a GEMM kernel (one workgroup per tile)
 * writes C, in order on `stream`. Same arguments as mk_gemm_ag_local. */
mk_status_t mk_gemm_ag_baseline(const void* A_local, const void* peers_A, int n_peers,
                                void* A_full, const void* B, void* C, int64_t Ms, int64_t N,
                                int64_t K, int rank, int c_dtype, void* stream);

/* G of mk_gemm_ag_local for these sizes on the current device (negative
 * mk_status_t on failure). */
int mk_ag_grid(int64_t Ms, int n_peers, int64_t N, int64_t K, int c_dtype);

/*
 * mk_flag_handoff -- microbenchmark and message-passing litmus of the tile-flag
 * protocol (Figure 2, item 1 of the thelatestinai.com page: a tile is handed to
 * communication by a readiness flag set once the tile is in GPU memory). Two
 * workgroups hand a flag back and forth `iters` times (1 .. 2^24), nothing else
 * in flight. Before each hand-off side 0 writes a data word (plain store); after
 * it side 1 reads the word (plain load) and counts values that are not the one
 * just published. flag_scope 0 = stores complete + relaxed flag store, consumer
 * invalidate at workgroup scope only (measured not to carry the data); 1 =
 * agent-scope release/acquire (MK_OPT_FLAG_SCOPE=1); 2 = the fused kernel's
 * default: stores complete + relaxed flag store, agent-scope acquire. cross_xcd
 * 0 = both workgroups on one XCD (the fused kernel's case), 1 = on two XCDs.
 * out: 16-byte-aligned device buffer of 5 uint64, written asynchronously on
 * `stream`: [0] 100 MHz ticks of all 2*iters hand-offs, [1] 1 if a wait passed
 * MK_OPT_SPIN_TIMEOUT_US (both sides then stop), [2], [3] the XCDs of the two
 * workgroups, [4] stale data reads. Uses the (device, stream) workspace's
 * control words.
 */
mk_status_t mk_flag_handoff(int iters, int flag_scope, int cross_xcd, void* stream, void* out);

/*
 * mk_mfma_peak -- the matrix-core ceiling the roofline is read against. Launches
 * n_workgroups workgroups of 256 threads (one per compute unit at most: 256
 * registers of accumulators per lane); each wave issues iters rounds of eight
 * independent bf16 v_mfma_f32_32x32x16 on register operands, 32768 flops each,
 * and no loads. Work: n_workgroups * 4 * 8 * iters * 32768 flops; the caller
 * times the call with events on `stream` (no timing inside).
 *   out : device buffer of n_workgroups * 256 floats (each lane's accumulator
 *         sum, written so that no product is dead); 4-byte aligned.
 *   iters 1 .. 2^24, n_workgroups 1 .. 65536, else MK_ERR_INVALID_ARG.
 */
mk_status_t mk_mfma_peak(int iters, int n_workgroups, void* out, void* stream);

/* Synchronizes `stream`, then returns and clears the device error word of that
 * stream's workspace and of the device's allocation-free workspace: MK_OK,
 * MK_ERR_TIMEOUT, MK_ERR_UNSUPPORTED or MK_ERR_INTERNAL (or MK_ERR_HIP if the
 * sync fails). */
mk_status_t mk_stream_status(void* stream);

/* Synchronizes the device and frees every workspace of `device`; the next call
 * recreates them zeroed. Use after an error. */
mk_status_t mk_workspace_reset(int device);

/*
 * mk_queue_plan -- how a persistent launch of `grid` workgroups on a device of
 * `cus` compute units queues its tiles, and the flag protocol that allows. A
 * kernel takes its queue from the hardware XCD id modulo the queue count. Tiles
 * are queued per XCD (cus / 32 queues on gfx950, 32 compute units per XCD) only
 * when cus is a multiple of 32 and grid a multiple of cus / 32 (at most 16
 * queues); then a tile is produced and consumed behind one L2 and the
 * requested protocol holds. Otherwise there is one queue, and flags use
 * agent-scope release and acquire (scope 1), which is correct across XCDs. The
 * kernels also check at run time that each queue is served by one XCD under
 * scope 0 (else MK_ERR_UNSUPPORTED from mk_stream_status). The same rule serves
 * mk_gemm_ar_local, mk_gemm_rs_local and mk_gemm_ag_local.
 *   flag_scope : the requested scope, 0 or 1 (MK_OPT_FLAG_SCOPE).
 *   n_xcd      : out, the number of queues.
 * Returns the scope used (0 or 1), or a negative mk_status_t for bad arguments.
 * Touches no GPU.
 */
int mk_queue_plan(int cus, int grid, int flag_scope, int* n_xcd);

/* G: workgroups of the fused kernel's persistent grid on `device` with its
 * large (256x256) tiles: one per compute unit. Returns a negative mk_status_t on
 * failure. */
int mk_num_workgroups(int device);

/* G for a call with these arguments on the current device: the resident
 * workgroup slots of the chosen tile shape (compute units times 1 for 256x256
 * tiles, times 2 for 128x128), but at most two per tile (with early reduce, see
 * MK_OPT_EARLY: one per tile, or two with MK_OPT_KSPLIT, plus one per reduce
 * unit of BM/64 rows), rounded
 * up to a multiple of the XCD count, for calls with few tiles. It depends on the
 * options in force at the time of the call. n_reduce_wg of that call
 * must lie in [0, G-1] or be MK_ADAPTIVE. Returns a negative mk_status_t on
 * failure. */
int mk_fused_grid(int64_t M, int64_t N, int64_t K, int n_peers, int peer_dtype, int c_dtype);

/* The schedule that mk_gemm_ar_local with these sizes, MK_ADAPTIVE and no
 * telemetry takes under the options in force: its tile shape as an
 * MK_OPT_TILE_SHAPE value, 1 = 256x256 and 2 = 128x128 (the persistent kernel;
 * with the default MK_OPT_INPLACE every tile reduced in place by the workgroup
 * that computed it, unless early reduce applies), 3 = 64x64 (one workgroup per
 * tile, in place), 4 and 5 = the wave-specialised kernel with 64x256 and 128x128
 * tiles. Returns a negative
 * mk_status_t on failure (no device included). */
int mk_fused_schedule(int64_t M, int64_t N, int64_t K, int n_peers, int peer_dtype, int c_dtype);

/* Tunables and debug switches (process-wide; read at each call). */
typedef enum {
  MK_OPT_SPIN_TIMEOUT_US = 0,   /* reducer flag-wait limit, microseconds (default 2000000) */
  MK_OPT_WITHHOLD_TILE = 1,     /* debug: compute skips publishing this tile (-1 = off) */
  MK_OPT_CTRL_PERIOD = 2,       /* controller runs every this many completed tiles (default 8) */
  MK_OPT_TILE_SHAPE = 3,        /* 0 = automatic, 1 = 256x256, 2 = 128x128, 3 = 64x64 (AllReduce
                                   only: each tile reduced in place by the workgroup that computed
                                   it; automatic for shapes with fewer 128x128 tiles than CUs),
                                   4 = wave-specialised (fused AllReduce only, without telemetry:
                                   64x256 tiles, one 384-thread workgroup per CU whose first four
                                   waves compute a tile while the other two reduce the tile
                                   before from LDS), 5 = the same with 128x128 tiles and four
                                   reducing waves (512 threads) (4 and 5:
                                   peer counts 0-4, 7, 8 and 15 of bfloat16, 0-4, 7 and 8 of
                                   float32; otherwise as 0). Automatic, with no reducer count,
                                   in-place policy, early reduce or k-split set, when the peer
                                   stream at HBM peak takes at least 1.8 times the GEMM at
                                   matrix-core peak and there are as many 64x256 tiles as CUs:
                                   64x256 tiles where the stream weighs most (see
                                   mk_fused_schedule), 128x128 otherwise */
  MK_OPT_FLAG_SCOPE = 4,        /* 0 = XCD-local flags (default: stores complete + relaxed flag store,
                                   agent-scope acquire), 1 = agent-scope release/acquire */
  MK_OPT_REDUCER_CAP = 5,       /* adaptive mode: most reducers while GEMM tiles remain (0 = derived) */
  MK_OPT_INPLACE = 6,           /* tiles per XCD reduced in place by the workgroup that computed them
                                   (the last ones of the XCD's queue; the others are handed to
                                   reducers through flags): -1 = automatic (default: every tile,
                                   or none with early reduce), 0 = none, n = the last n of each
                                   queue; -2 = dynamic hand-over: a tile is reduced in place when
                                   its GEMM ends if fewer workgroups than the reducer target are
                                   streaming a reduce on its XCD (or no GEMM tile is left), else
                                   published for reducers; the target (n_reduce_wg, or the
                                   controller's with MK_ADAPTIVE) counts streaming workgroups */
  MK_OPT_EARLY = 7,             /* early reduce: a reducer may take a unit whose tile is still being
                                   computed and sums that unit's peers (into LDS) while it waits for
                                   the tile's flag. -1 = automatic (default: on when every tile and
                                   every reduce unit gets a workgroup of its own in one round, e.g.
                                   few-tile decode shapes; the grid then holds one workgroup per
                                   tile plus one per unit, and tiles are handed over rather than
                                   reduced in place), 0 = off, 1 = on. Peer counts 1-4, 7, 8, 15. */
  MK_OPT_KSPLIT = 8,            /* with early reduce and every tile handed over: each tile computed
                                   as two k-halves (two workgroups, two fp32 partials, a flag each;
                                   the reducer adds P0 + P1 to the peer sum). -1 = automatic (on
                                   when K is a multiple of 64, at least 512, and two items per tile
                                   plus the reduce units fit one round), 1 = off, 2 = on (K a
                                   multiple of 64). The fp32 rounding of P0 + P1 differs from one
                                   k-loop, so C can differ from the baseline in the last bit. */
  MK_OPT_STREAM_CU_SPLIT = 9,   /* mk_gemm_ar_two_stream: compute units given to the reduce stream
                                   when the two streams are CU-masked; the GEMM stream gets the
                                   rest. 0 = no masks (default: both streams share the chip). R > 0
                                   must be below the device's compute units and a multiple of 8
                                   per 32-unit mask word (64 on a 256-unit MI355X), so that every
                                   word, whichever XCD its units sit on, gives the reduce stream
                                   the same share; checked at the call (MK_ERR_INVALID_ARG). Each
                                   word's top R/words bits go to the reduce stream. */
  MK_OPT_STATIC_TILES = 10      /* 256x256 tiles all reduced in place with more tiles than one round
                                   of workgroups (the default schedule of compute-bound shapes,
                                   without telemetry): 2 = the in-place kernel, which deals each
                                   XCD's range of tiles to its workgroups in a fixed order and
                                   keeps no claim, flag or counter, with eight waves per
                                   workgroup where the tile-end reduce fits two waves per SIMD
                                   (bfloat16 peer counts 0-4, 7, 8, 15; float32 0-4, 7), else
                                   four (default); 1 = the in-place kernel with four waves; 0 =
                                   the persistent kernel with per-XCD tile claims. All give the
                                   same bits. With 2, the baselines' GEMM kernel also takes the
                                   eight-wave 256x256 tile when there are more tiles than
                                   compute units. */
} mk_option_t;
mk_status_t mk_set_option(int option, int64_t value);
int64_t mk_get_option(int option);

/* Host copy of the controller rule that the fused kernel runs on the device;
 * exported so that its behaviour can be simulated on the CPU.
 *   G        workgroups, T tiles
 *   T_r      tiles handed to reducers (T minus those reduced in place)
 *   computed tiles computed; reduced: handed-over tiles reduced
 *   busy_c   summed compute time (in-place tiles whole); busy_r summed reduce
 *            time of handed-over tiles, without flag waits
 *   seed_x   the host's initial reducer fraction in [0,1]
 *   current  the target now in force
 *   cap      most reducers while GEMM tiles remain (< 0: G-1; 0: none)
 * Returns the new target. */
int mk_controller_eval(int G, int T, int T_r, int computed, int reduced, uint64_t busy_c,
                       uint64_t busy_r, float seed_x, int current, int cap);

const char* mk_status_string(int status);
const char* mk_last_error(void);
int mk_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MK_H_ */
