// mk_kernels.hip -- the fused persistent GEMM+AllReduce kernel (one GPU's share)
// and the two-kernel baseline, for gfx950.
//
// Fused schedule: Figure 1(c) and Figure 2 of the thelatestinai.com page of
// "mKernel: Fast Multi-GPU, Multi-Node Fused Kernels": a persistent kernel whose
// workgroups take compute or communication roles; compute publishes each
// finished tile with a readiness flag, communication consumes it as soon as it
// is ready, and a controller retunes the number of communication workgroups.
// Baseline: Figure 1(a)/(b)'s kernel-boundary schedule reduced to one GPU: a GEMM
// kernel writes every partial tile, then a reduce kernel runs.
#include "mk_kernels.h"

#include "mk_controller.h"
#include "mk_device.h"

namespace mk {

// ------------------------------------------------------------ workspace slots

__device__ __forceinline__ int* slot32(unsigned long long* s, int i) {
  return (int*)(s + (size_t)i * kSlotWords);
}
__device__ __forceinline__ unsigned long long* slot64(unsigned long long* s, int i) {
  return s + (size_t)i * kSlotWords;
}

__device__ __forceinline__ int* xslot(unsigned long long* s, int x, int w) {
  return slot32(s, S_XCD_BASE + x * kXcdWords + w);
}
__device__ __forceinline__ unsigned long long* xslot64(unsigned long long* s, int x, int w) {
  return slot64(s, S_XCD_BASE + x * kXcdWords + w);
}

// Sum of a per-XCD word over the n_xcd XCDs (all loads issued before any add).
__device__ __forceinline__ int sum_xcd32(unsigned long long* S, int n_xcd, int w) {
  int v[kMaxXcd];
#pragma unroll
  for (int x = 0; x < kMaxXcd; ++x) v[x] = x < n_xcd ? load_relaxed(xslot(S, x, w)) : 0;
  int t = 0;
#pragma unroll
  for (int x = 0; x < kMaxXcd; ++x) t += v[x];
  return t;
}
__device__ __forceinline__ unsigned long long sum_xcd64(unsigned long long* S, int n_xcd, int w) {
  unsigned long long v[kMaxXcd];
#pragma unroll
  for (int x = 0; x < kMaxXcd; ++x)
    v[x] = x < n_xcd ? __hip_atomic_load(xslot64(S, x, w), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                     : 0ull;
  unsigned long long t = 0;
#pragma unroll
  for (int x = 0; x < kMaxXcd; ++x) t += v[x];
  return t;
}

__device__ __forceinline__ int current_target(unsigned long long* S, int epoch, int init_target) {
  unsigned long long w =
      __hip_atomic_load(slot64(S, S_TARGET), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if ((int)(w >> 32) == epoch) return (int)(w & 0xFFFFFFFFu);
  return init_target;
}

__device__ __forceinline__ void raise_error(unsigned long long* S, int code) {
  atomicCAS(slot32(S, S_ERROR), 0, code);
  __hip_atomic_store(slot32(S, S_ABORT), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The XCD-local flag protocol needs every workgroup of a queue to run on one
// XCD (the host's queue_plan arranges that for the device's known layout). The
// first workgroup of queue x records its hardware XCD id; a workgroup of
// another XCD on the same queue stops the kernel with MK_ERR_UNSUPPORTED
// instead of exchanging tiles through two L2s. Thread 0 only.
__device__ __forceinline__ bool same_xcd_queue(unsigned long long* S, int x, int hw_xcd) {
  const int me = hw_xcd + 1;
  const int prev = atomicCAS(xslot(S, x, X_PHYS), 0, me);
  if (prev == 0 || prev == me) return true;
  raise_error(S, MK_ERR_UNSUPPORTED);
  return false;
}

// One controller evaluation (thread 0 of the workgroup that wins the try-lock).
// Takes its inputs by value: the kernel's argument block must not escape to
// memory, or every pointer read from it loses its global address space. Inlined:
// a call would make the kernel save its live registers around every call site.
__device__ __forceinline__ void controller_step(unsigned long long* S, mk_telemetry_t* tel, int G,
                                             int T, int T_r, int epoch, int init_target,
                                             float seed_x, int cap, int rsplit, int n_xcd,
                                             int dyn) {
  if (atomicCAS(slot32(S, S_LOCK), 0, 1) != 0) return;
  int c = sum_xcd32(S, n_xcd, X_COMPUTED);
  // tiles reduced (reduce units -> tiles): every one when the target counts
  // streaming workgroups, else the handed-over ones (less those done in place)
  int r = sum_xcd32(S, n_xcd, X_REDUCED) / rsplit - (dyn ? 0 : sum_xcd32(S, n_xcd, X_INPLACE));
  unsigned long long bc = sum_xcd64(S, n_xcd, X_BUSY_C);
  unsigned long long br = sum_xcd64(S, n_xcd, X_BUSY_R);
  int cur = current_target(S, epoch, init_target);
  int nt = controller_rule(G, T, T_r, c, r, bc, br, seed_x, cur, cap);
  if (nt != cur) {
    unsigned long long w = ((unsigned long long)(unsigned)epoch << 32) | (unsigned)nt;
    __hip_atomic_store(slot64(S, S_TARGET), w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    atomicAdd(slot32(S, S_UPDATES), 1);
  }
  if (tel) {
    int i = atomicAdd(slot32(S, S_NTRACE), 1);
    if (i < MK_TRACE_CAP) {
      mk_trace_entry_t e;
      e.t = ticks();
      e.computed = c;
      e.reduced = r;
      e.target = nt;
      e.spare = sum_xcd32(S, n_xcd, X_STREAM);
      tel->trace[i] = e;
    }
  }
  // Unlock once this thread's stores (target, trace) have completed; an
  // agent-scope release would write back the whole XCD L2 at every update.
  wait_stores();
  __hip_atomic_store(slot32(S, S_LOCK), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

enum { K_EXIT = 0, K_COMPUTE = 1, K_REDUCE = 2 };

// GEMM+ReduceScatter share, a reduce unit of a handed-over tile: rows
// [r0, r0+rows) whose fp32 partial is in the workspace (all M rows). Owned rows
// are reduced into C, the others rounded to the peer type into send.
template <int OCC, typename PT, typename CT>
__device__ __forceinline__ void rs_unit(const FusedArgs& a, int64_t r0, int64_t n0, int rows,
                                        int cols) {
  const int64_t r1 = r0 + rows;  // rows <= 0: nothing
  const int64_t lo = r1 < a.own0 ? r1 : a.own0, hi = r1 < a.own1 ? r1 : a.own1;
  const int64_t o0 = r0 > lo ? r0 : lo;  // owned rows [o0, o1)
  const int64_t o1 = o0 > hi ? o0 : hi;
  const int64_t own_rows = a.own1 - a.own0;
  reduce_region<OCC, PT, PT>(a.P, (const PT*)nullptr, 0, (PT*)a.send, a.M, a.N, r0, n0,
                             (int)(o0 - r0), cols);
  if (o1 > o0)  // the workspace shifted so that its row o0 is row o0 - own0 of C
    reduce_region<OCC, PT, CT>(a.P + a.own0 * a.N, (const PT*)a.peers, a.n_peers, (CT*)a.C,
                               own_rows, a.N, o0 - a.own0, n0, (int)(o1 - o0), cols);
  reduce_region<OCC, PT, PT>(a.P, (const PT*)nullptr, 0, (PT*)a.send, a.M, a.N, o1, n0,
                             (int)(r1 - o1), cols);
}

// GEMM+ReduceScatter share, one band of a tile's rows [r0, r0+rows) whose fp32
// partial sits in LDS (pitch LP). Tiles handled in place hold no owned row (the
// tile rows with owned rows are handed over), so the band is published: rounded
// to the peer type into send, which the rows' owners receive as a peer partial.
template <typename PT>
__device__ __forceinline__ void rs_band(const FusedArgs& a, const char* band, int64_t LP,
                                        int64_t r0, int64_t n0, int rows, int cols) {
  copy_region_lds<PT>(band, LP, (PT*)a.send, a.N, r0, n0, rows, cols);
}



// Persistent fused kernel. Tiles [start_x, start_x + cnt_x) belong to XCD x: only
// workgroups running on XCD x compute or reduce them, so a tile's partial is
// produced and consumed behind the same L2. A tile's reduce is split into
// RSPLIT row-slab units. In each XCD, workgroups whose arrival rank is below
// that XCD's share of the reducer target prefer reducing; the others prefer
// computing. A reducer reserves the next unit when its tile is finished (or no
// GEMM tile is left) and computes a tile otherwise; a reserved unit whose tile
// nobody has claimed yet makes its holder compute that far. Compute workgroups
// reserve units once no GEMM tile is left (draining).
// A tile reduced in place, straight from the accumulators of the workgroup that
// computed it: the fp32 tile goes through LDS (free after the GEMM's last barrier)
// in passes, each summed in the order of every other path. All threads (NW
// waves); with eight waves two share a SIMD, and the reduce rings take the
// register budget of two workgroups per compute unit.
template <class Cfg>
constexpr int ring_occ() {
  return Cfg::NW == 8 ? 2 : Cfg::OCC;
}
template <class Cfg, typename PT, typename CT>
__device__ __forceinline__ void inplace_tile(const GemmTile<Cfg>& g, char* lds, const PT* peers,
                                             int n_peers, CT* C, int64_t M, int64_t N, int64_t m0,
                                             int64_t n0) {
  const int cols = (int)(N - n0 < Cfg::BN ? N - n0 : Cfg::BN);
  constexpr int BAND = GemmTile<Cfg>::BAND;
  auto pass = [&](auto pass_c) {
    constexpr int PASS = decltype(pass_c)::value;
    g.template stage_pass_lds<PASS>(lds);
    __syncthreads();
    if constexpr (GemmTile<Cfg>::NPASS == 1 && 2 * BAND == Cfg::BM) {
      const int rows = (int)(M - m0 < Cfg::BM ? M - m0 : Cfg::BM);
      reduce_region_lds<ring_occ<Cfg>(), PT, CT, Cfg::NW * 64>(lds, Cfg::BN, peers, n_peers, C, M,
                                                               N, m0, n0, rows, cols);
    } else {
#pragma unroll
      for (int wm = 0; wm < 2; ++wm) {
        const int64_t r0 = m0 + wm * Cfg::WM + PASS * BAND;
        const int rows = (int)(M - r0 < BAND ? M - r0 : BAND);  // <= 0 past the edge
        reduce_region_lds<ring_occ<Cfg>(), PT, CT, Cfg::NW * 64>(
            lds + wm * BAND * Cfg::BN * 4, Cfg::BN, peers, n_peers, C, M, N, r0, n0, rows, cols);
      }
    }
    __syncthreads();
  };
  pass(std::integral_constant<int, 0>{});
  if constexpr (GemmTile<Cfg>::NPASS > 1) pass(std::integral_constant<int, 1>{});
}

// DYN: dynamic hand-over (a compile-time variant, so that the default schedule's
// code is not shaped by it).
template <class Cfg, typename PT, typename CT, bool DYN>
__global__ __launch_bounds__(kThreads, Cfg::OCC) void fused_kernel(FusedArgs a) {
  __shared__ __align__(1024) char lds[Cfg::LDS_BYTES];
  __shared__ int s_kind, s_tile, s_part, s_ok, s_last, s_inpl;
  const int tid = threadIdx.x;
  unsigned long long* S = a.slots;
  const PT* peers = (const PT*)a.peers;
  CT* C = (CT*)a.C;
  if (a.one_tile) {
    // Every tile reduced in place, at least one workgroup per tile: the tile
    // comes from the workgroup index (XCD-aware like the baseline GEMM kernel),
    // and no claim, counter, flag or controller is involved.
    const int b = blockIdx.x;
    if (b >= a.T) return;  // workgroups beyond the tiles (a grid of at least one per XCD)
    const int t = a.G == a.T && a.n_xcd > 1 && a.T % a.n_xcd == 0
                      ? (b % a.n_xcd) * (a.T / a.n_xcd) + b / a.n_xcd
                      : b;
    int tm, tn;
    fused_tile_coords(t, a.tiles_m, a.tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * Cfg::BM, n0 = (int64_t)tn * Cfg::BN;
    GemmTile<Cfg> g;
    g.run(a.A, a.B, a.M, a.N, a.K, m0, n0, lds);
    inplace_tile<Cfg, PT, CT>(g, lds, peers, a.n_peers, C, a.M, a.N, m0, n0);
    return;
  }
  const unsigned long long t_begin = ticks();

  // thread 0 state
  const int hw_xcd = xcc_id();
  const int x = hw_xcd % a.n_xcd;
  const int q0 = (int)(((int64_t)x * a.T) / a.n_xcd);
  const int cnt = (int)(((int64_t)(x + 1) * a.T) / a.n_xcd) - q0;
  int rank = -1, last_kind = -1, held = -1;  // held: reserved reduce unit of this XCD
  bool flag_seen = false;  // thread 0: the claimed unit's flag was already read as set
  unsigned long long t_busy = 0;  // thread 0: a reduce unit's busy ticks, less its end tick
  // ReduceScatter share: the XCD's queue starts with its share of the tiles in
  // the tile rows that hold owned rows; those are handed to reducers, the rest
  // (published rows only) are handled in place.
  int rs_ox0 = 0, rs_ox = 0;
  if (a.rs) rs_share(x, a.n_xcd, a.T, (a.tmo1 - a.tmo0) * a.tiles_n, rs_ox0, rs_ox);
  // The last n_in tiles of the XCD's queue are reduced in place by the workgroup
  // that computes them: no partial goes through memory, no flag is involved.
  const int n_in = a.rs ? cnt - rs_ox
                        : xcd_inplace(cnt, a.n_inplace,
                                      inplace_supported(Cfg::OCC, (int)sizeof(PT), a.n_peers));
  const int published = cnt - n_in;
  // Early reduce: a unit's peers are summed into LDS before its flag is read.
  static_assert(Cfg::BM / Cfg::RSPLIT * Cfg::BN * 4 <= Cfg::LDS_BYTES, "peer sum of a unit in LDS");
  const bool early = a.early && a.n_peers > 0 &&
                     inplace_supported(Cfg::OCC, (int)sizeof(PT), a.n_peers);
  // K-split: compute item i of the XCD's queue is k-half i % KS of tile i / KS. A
  // tile counts as claimed once all of its items are.
  const int KS = a.ksplit > 1 ? a.ksplit : 1;
  const int items = cnt * KS;
  // Dynamic hand-over: every tile of the queue may be handed over, so its reduce
  // units are indexed over the whole queue; a tile reduced in place has its flag
  // set to -epoch, and its units are skipped.
  const bool inpl_ok = inplace_supported(Cfg::OCC, (int)sizeof(PT), a.n_peers);
  unsigned long long w_start = 0;  // thread 0: start of a wait for an undecided tile

  for (;;) {
    if constexpr (DYN) if (tid == 0) {
      // The reducer target counts workgroups streaming a reduce (in place or a
      // handed-over unit). A tile is handed over only when its GEMM ends with
      // every streaming slot of the XCD taken; it then gets the next slot of the
      // XCD's publication list. A workgroup takes a published unit when a
      // streaming slot is free, computes a GEMM tile otherwise, and drains the
      // published units once no GEMM tile is left; it leaves when every tile of
      // the queue is done and every published unit is taken.
      int kind = K_EXIT, tile = -1;
      int* rnext = xslot(S, x, X_REDUCE_NEXT);
      int* cnext = xslot(S, x, X_COMPUTE_NEXT);
      flag_seen = false;
      for (;;) {
        const int abort = load_relaxed(slot32(S, S_ABORT));
        const unsigned long long tw =
            __hip_atomic_load(slot64(S, S_TARGET), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int cn = load_relaxed(cnext);
        const int rn = load_relaxed(rnext);
        const int st = load_relaxed(xslot(S, x, X_STREAM));
        const int done = load_relaxed(xslot(S, x, X_COMPUTED));
        int np = load_relaxed(xslot(S, x, X_PUB));
        // Once every tile is computed the list is final, but the load above may
        // have been served before the one of `done`: load it again, issued after
        // `done` has returned (the branch waits for it).
        if (done >= cnt) np = load_relaxed(xslot(S, x, X_PUB));
        if (rank < 0) {
          rank = atomicAdd(xslot(S, x, X_ARRIVE), 1);
          if (a.flag_scope == 0 && !same_xcd_queue(S, x, hw_xcd)) break;
        }
        if (abort) break;
        const int target = (int)(tw >> 32) == a.epoch ? (int)(tw & 0xFFFFFFFFu) : a.init_target;
        const int tx = target / a.n_xcd + (x < target % a.n_xcd ? 1 : 0);
        const int avail = np * Cfg::RSPLIT;  // units of the published tiles
        if (held >= 0) {
          const int s = held / Cfg::RSPLIT;
          if (s < np) {
            const unsigned long long wd = __hip_atomic_load(a.pub + q0 + s, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT);
            if ((int)(wd >> 32) == a.epoch) {
              kind = K_REDUCE;
              tile = (int)(wd & 0xFFFFFFFFu);
              s_part = held % Cfg::RSPLIT;
              flag_seen = true;
              held = -1;
              w_start = 0;
              break;
            }
          } else if (done >= cnt) {
            held = -1;  // every tile is done and this unit was never published
            break;
          } else if (cn < cnt) {
            const int i = atomicAdd(cnext, 1);  // compute while the unit is not published
            if (i < cnt) {
              kind = K_COMPUTE;
              tile = q0 + i;
              break;
            }
          }
          // the slot is taken but its word not yet written, or the last tiles
          // are still computing: wait (bounded)
          if (w_start == 0) w_start = ticks();
          if (ticks() - w_start > a.spin_limit) {
            raise_error(S, MK_ERR_TIMEOUT);
            break;
          }
          backoff_sleep(1);
          continue;
        }
        w_start = 0;
        if (rn < avail && (st < tx || cn >= cnt)) {
          held = atomicAdd(rnext, 1);
          continue;
        }
        if (cn < cnt) {
          const int i = atomicAdd(cnext, 1);
          if (i < cnt) {
            kind = K_COMPUTE;
            tile = q0 + i;
            break;
          }
          continue;
        }
        if (done < cnt) {  // no GEMM left to start; tiles still computing may be published
          if (rn < avail) {
            held = atomicAdd(rnext, 1);
            continue;
          }
          if (w_start == 0) w_start = ticks();
          if (ticks() - w_start > a.spin_limit) {
            raise_error(S, MK_ERR_TIMEOUT);
            break;
          }
          backoff_sleep(2);
          continue;
        }
        if (rn < avail) {
          held = atomicAdd(rnext, 1);
          continue;
        }
        break;
      }
      if (kind != K_EXIT) {
        if (last_kind >= 0 && kind != last_kind) atomicAdd(xslot(S, x, X_SWITCHES), 1);
        last_kind = kind;
      }
      s_kind = kind;
      s_tile = tile;
      if (kind == K_COMPUTE) s_part = 0;
    }
    if (!DYN && tid == 0) {
      int kind = K_EXIT, tile = -1, part = 0;
      bool off_role = false;
      const int units = published * Cfg::RSPLIT;  // unit r: slab r % RSPLIT of tile r / RSPLIT
      int* rnext = xslot(S, x, X_REDUCE_NEXT);
      int* cnext = xslot(S, x, X_COMPUTE_NEXT);
      flag_seen = false;
      // Every pass claims work or leaves; nothing here waits for other
      // workgroups. The state every decision reads is loaded in one round trip
      // (independent loads), and a pass ends with at most two atomics.
      for (;;) {
        const int abort = load_relaxed(slot32(S, S_ABORT));
        const unsigned long long tw =
            __hip_atomic_load(slot64(S, S_TARGET), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int cn = load_relaxed(cnext);  // compute items claimed (a lower bound)
        const int rn = load_relaxed(rnext);  // next reduce unit
        // The arrival rank is taken in the first pass, in the same round trip
        // as the loads above.
        if (rank < 0) {
          rank = atomicAdd(xslot(S, x, X_ARRIVE), 1);
          if (a.flag_scope == 0 && !same_xcd_queue(S, x, hw_xcd)) break;
        }
        if (abort) break;
        const int target = (int)(tw >> 32) == a.epoch ? (int)(tw & 0xFFFFFFFFu) : a.init_target;
        const int tx = target / a.n_xcd + (x < target % a.n_xcd ? 1 : 0);
        const bool pref_reduce = rank < tx;
        if (held >= 0) {
          // A reserved unit is reduced once a compute workgroup has claimed its
          // tile (that workgroup is running, so the flag will be set). Until
          // then this workgroup computes the next tile itself: that claim cannot
          // fail while the reserved tile is unclaimed, so the XCD always makes
          // progress.
          if ((held / Cfg::RSPLIT + 1) * KS <= cn) {
            kind = K_REDUCE;
            tile = q0 + held / Cfg::RSPLIT;
            part = held % Cfg::RSPLIT;
            off_role = !pref_reduce;
            held = -1;
            break;
          }
          const int i = atomicAdd(cnext, 1);
          if (i < items) {
            kind = K_COMPUTE;
            tile = q0 + i / KS;
            part = i % KS;
            off_role = pref_reduce;
            break;
          }
          continue;  // the tile was claimed meanwhile
        }
        if (!pref_reduce && cn < items) {
          const int i = atomicAdd(cnext, 1);
          if (i < items) {
            kind = K_COMPUTE;
            tile = q0 + i / KS;
            part = i % KS;
            break;
          }
        }
        if (rn >= units) {
          // Every reduce unit is taken. Tiles reduced in place have no units, so
          // GEMM tiles may remain: take one before leaving.
          if (pref_reduce && cn < items) {
            const int i = atomicAdd(cnext, 1);
            if (i < items) {
              kind = K_COMPUTE;
              tile = q0 + i / KS;
              part = i % KS;
              off_role = true;
            }
          }
          break;
        }
        int fl = 0;
        if (pref_reduce && cn < items) {
          // GEMM tiles are left: reserve the next unit only if its tile is
          // finished (or, with early reduce, being computed: its peers are
          // summed meanwhile), else compute rather than wait for its flag.
          const int ft = (q0 + rn / Cfg::RSPLIT) * KS;
          fl = load_relaxed(a.flags + ft);
          for (int h = 1; h < KS; ++h)
            if (load_relaxed(a.flags + ft + h) != a.epoch) fl = 0;
          if (fl != a.epoch && !(early && (rn / Cfg::RSPLIT + 1) * KS <= cn)) {
            const int i = atomicAdd(cnext, 1);
            if (i < items) {
              kind = K_COMPUTE;
              tile = q0 + i / KS;
              part = i % KS;
              off_role = true;
              break;
            }
          }
        }
        // Reserve the next reduce unit (a fetch-add always succeeds, unlike a
        // compare-and-swap that 32 workgroups of an XCD would retry in turn).
        held = atomicAdd(rnext, 1);
        if (held >= units) {
          held = -1;
          break;
        }
        if ((held / Cfg::RSPLIT + 1) * KS <= cn) {
          kind = K_REDUCE;
          tile = q0 + held / Cfg::RSPLIT;
          part = held % Cfg::RSPLIT;
          off_role = !pref_reduce;
          // the flag read above covers this unit when it is the same tile
          flag_seen = fl == a.epoch && held / Cfg::RSPLIT == rn / Cfg::RSPLIT;
          held = -1;
          break;
        }
      }
      if (kind != K_EXIT) {
        if (last_kind >= 0 && kind != last_kind) atomicAdd(xslot(S, x, X_SWITCHES), 1);
        last_kind = kind;
        if (off_role) atomicAdd(xslot(S, x, kind == K_REDUCE ? X_RBC : X_CBR), 1);
      }
      s_kind = kind;
      s_tile = tile;
      s_part = part;
    }
    __syncthreads();
    const int kind = s_kind, tile = s_tile, part = s_part;
    if (kind == K_EXIT) break;
    int tm, tn;
    if (a.rs)
      rs_tile_coords(tile - q0, q0, rs_ox0, rs_ox, a.tiles_m, a.tiles_n, a.tmo0, a.tmo1, tm, tn);
    else
      fused_tile_coords(tile, a.tiles_m, a.tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * Cfg::BM, n0 = (int64_t)tn * Cfg::BN;

    if (kind == K_COMPUTE) {
      const unsigned long long t0 = ticks();
      // Nothing of the previous task is still needed; waiting for all of this
      // wave's loads here (a wait the compiler tracks) lets it start the GEMM
      // with no load outstanding, so it adds no waits to the k-loop.
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      GemmTile<Cfg> g;
      if (KS > 1) {  // k-half `part` of the tile: A and B advanced, A's pitch K
        const int64_t kh = a.K / KS, k0 = kh * part;
        g.run(a.A + k0, a.B + k0 * a.N, a.M, a.N, kh, m0, n0, lds, NoGate(), a.K);
      } else {
        g.run(a.A, a.B, a.M, a.N, a.K, m0, n0, lds);
      }
      const unsigned long long t_gemm = DYN ? ticks() : 0;
      if constexpr (DYN) {
        // In place while a streaming slot of the XCD is free or no GEMM tile is
        // left to start; otherwise hand the tile over and compute the next one.
        if (tid == 0) {
          const unsigned long long tw = __hip_atomic_load(slot64(S, S_TARGET), __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT);
          const int target =
              (int)(tw >> 32) == a.epoch ? (int)(tw & 0xFFFFFFFFu) : a.init_target;
          const int tx = target / a.n_xcd + (x < target % a.n_xcd ? 1 : 0);
          const int st = load_relaxed(xslot(S, x, X_STREAM));
          const int cn = load_relaxed(xslot(S, x, X_COMPUTE_NEXT));
          const int inpl = inpl_ok && (cn >= cnt || st < tx) && tile != a.withhold_tile;
          if (inpl) atomicAdd(xslot(S, x, X_STREAM), 1);
          s_inpl = inpl;
        }
        __syncthreads();
      }
      if (DYN ? s_inpl != 0 : tile - q0 >= published) {
        // In place: the partial goes through LDS (freed by the GEMM's last
        // barrier) in passes, each summed in the same order as a reducer would.
        const int cols = (int)(a.N - n0 < Cfg::BN ? a.N - n0 : Cfg::BN);
        auto pass = [&](auto pass_c) {
          constexpr int PASS = decltype(pass_c)::value;
          constexpr int BAND = GemmTile<Cfg>::BAND;
          g.template stage_pass_lds<PASS>(lds);
          __syncthreads();
          if constexpr (GemmTile<Cfg>::NPASS == 1 && 2 * BAND == Cfg::BM) {
            // the whole tile is in LDS, its rows in order: one region
            const int rows = (int)(a.M - m0 < Cfg::BM ? a.M - m0 : Cfg::BM);
            if (a.rs)
              rs_band<PT>(a, lds, Cfg::BN, m0, n0, rows, cols);
            else
              reduce_region_lds<Cfg::OCC, PT, CT>(lds, Cfg::BN, peers, a.n_peers, C, a.M, a.N,
                                                  m0, n0, rows, cols);
          } else {
#pragma unroll
            for (int wm = 0; wm < 2; ++wm) {
              const int64_t r0 = m0 + wm * Cfg::WM + PASS * BAND;
              const int rows = (int)(a.M - r0 < BAND ? a.M - r0 : BAND);  // <= 0 past the edge
              const char* band = lds + wm * BAND * Cfg::BN * 4;
              if (a.rs)
                rs_band<PT>(a, band, Cfg::BN, r0, n0, rows, cols);
              else
                reduce_region_lds<Cfg::OCC, PT, CT>(band, Cfg::BN, peers, a.n_peers, C, a.M, a.N,
                                                    r0, n0, rows, cols);
            }
          }
          __syncthreads();
        };
        pass(std::integral_constant<int, 0>{});
        if constexpr (GemmTile<Cfg>::NPASS > 1) pass(std::integral_constant<int, 1>{});
        if (tid == 0) {
          const unsigned long long t1 = ticks();
          if constexpr (DYN) {
            // the GEMM counts as compute work, the reduce as streaming work
            atomicAdd(xslot(S, x, X_STREAM), -1);
            int done = atomicAdd(xslot(S, x, X_COMPUTED), 1) + 1;
            atomicAdd(xslot64(S, x, X_BUSY_C), t_gemm - t0);
            atomicAdd(xslot64(S, x, X_BUSY_R), t1 - t_gemm);
            atomicAdd(xslot(S, x, X_REDUCED), Cfg::RSPLIT);
            atomicAdd(xslot(S, x, X_INPLACE), 1);
            if (a.adaptive && (done % a.ctrl_period) == 0)
              controller_step(S, a.tel, a.G, a.T, a.T_r, a.epoch, a.init_target, a.seed_x,
                              a.reducer_cap, Cfg::RSPLIT, a.n_xcd, 1);
          } else {
            // the whole tile counts as compute work for the controller
            int done = atomicAdd(xslot(S, x, X_COMPUTED), 1) + 1;
            atomicAdd(xslot64(S, x, X_BUSY_C), t1 - t0);
            atomicAdd(xslot(S, x, X_REDUCED), Cfg::RSPLIT);
            atomicAdd(xslot(S, x, X_INPLACE), 1);
            if (a.adaptive && KS == 1 && (done % a.ctrl_period) == 0)
              controller_step(S, a.tel, a.G, a.T, a.T_r, a.epoch, a.init_target, a.seed_x,
                              a.reducer_cap, Cfg::RSPLIT, a.n_xcd, 0);
          }
        }
        __syncthreads();
        continue;
      }
      g.store_partial(a.P + (KS > 1 ? part * a.M * a.N : 0), a.M, a.N, m0, n0);
      // with telemetry: ticks from here (stores issued) to the flag store
      const unsigned long long tp0 = a.tel && tid == 0 ? ticks() : 0ull;
      wait_stores();    // this wave's partial stores have reached the L2
      __syncthreads();  // ... and so have every other wave's
      if (tid == 0) {
        if constexpr (DYN) {
          // the next slot of the XCD's publication list; the slot count is raised
          // before the computed count, so a queue whose tiles are all computed
          // has its final list
          const int s = atomicAdd(xslot(S, x, X_PUB), 1);
          const unsigned long long wd = ((unsigned long long)(unsigned)a.epoch << 32) | (unsigned)tile;
          unsigned long long* wp = a.pub + q0 + s;
          if (tile == a.withhold_tile) {
          } else if (a.flag_scope == 0) {
            __hip_atomic_store(wp, wd, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          } else {
            __hip_atomic_store(wp, wd, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
          }
        } else if (tile != a.withhold_tile) {
          int* fp = a.flags + tile * KS + part;
          if (a.flag_scope == 0) store_flag(fp, a.epoch);
          else publish_flag_agent(fp, a.epoch);
        }
        if (a.tel) {
          atomicAdd(xslot64(S, x, X_PUB_T), ticks() - tp0);
          atomicAdd(xslot(S, x, X_NPUB), 1);
        }
        int done = atomicAdd(xslot(S, x, X_COMPUTED), 1) + 1;  // this XCD's count
        atomicAdd(xslot64(S, x, X_BUSY_C), ticks() - t0);
        // (with a k-split the call fits one round of workgroups: no controller)
        if (a.adaptive && KS == 1 && (done % a.ctrl_period) == 0)
          controller_step(S, a.tel, a.G, a.T, a.T_r, a.epoch, a.init_target, a.seed_x,
                          a.reducer_cap, Cfg::RSPLIT, a.n_xcd, DYN ? 1 : 0);
      }
    } else {
      constexpr int SLAB = Cfg::BM / Cfg::RSPLIT;
      const int64_t r0 = m0 + (int64_t)part * SLAB;
      const int rows = (int)(a.M - r0 < SLAB ? a.M - r0 : SLAB);  // <= 0 past a ragged edge
      const int cols = (int)(a.N - n0 < Cfg::BN ? a.N - n0 : Cfg::BN);
      const unsigned long long t0 = ticks();
      if (DYN && tid == 0) atomicAdd(xslot(S, x, X_STREAM), 1);
      if (early) {
        // phase 1: the peers need no flag
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no load of the last task in flight
        reduce_region_peers_lds<Cfg::OCC, PT>(lds, Cfg::BN, peers, a.n_peers, a.M, a.N, r0, n0,
                                              rows, cols);
      }
      if (tid == 0) {
        const unsigned long long w0 = ticks();
        int ok = 1, backoff = 1;
        // the tile's flags (one per k-part), each polled until set
        for (int h = 0; h < KS && !flag_seen && ok; ++h) {
          while (load_relaxed(a.flags + tile * KS + h) != a.epoch) {
            if (load_relaxed(slot32(S, S_ABORT))) {
              ok = 0;
              break;
            }
            if (ticks() - w0 > a.spin_limit) {
              raise_error(S, MK_ERR_TIMEOUT);
              ok = 0;
              break;
            }
            backoff_sleep(backoff);
            backoff = backoff < 4 ? backoff * 2 : 4;
          }
        }
        const unsigned long long ws = ticks();  // every flag of the unit seen set
        // The partial must not come from a stale L1 copy: with lines that can
        // hold two units' rows (or agent-scope flags) acquire at agent scope;
        // otherwise this compute unit has never read the unit's lines in this
        // call, so its L1 holds no copy of them (see mk_device.h).
        if (a.flag_scope != 0 || a.shared_lines) acquire_fence_agent();
        const unsigned long long w1 = ticks();
        atomicAdd(xslot64(S, x, X_WAIT_R), w1 - w0);
        if (a.tel && ok) {
          atomicAdd(xslot64(S, x, X_ACQ_T), w1 - ws);
          atomicAdd(xslot(S, x, X_NACQ), 1);
        }
        s_ok = ok;
        // busy time: phase 1 plus what follows the wait
        t_busy = (w0 - t0) - w1;
      }
      __syncthreads();  // also: phase 1's LDS writes are done
      if (!s_ok) break;
      if (early && KS == 2)
        reduce_region_finish_parts<2, CT>(a.P, a.M * a.N, lds, Cfg::BN, C, a.N, r0, n0, rows, cols);
      else if (KS > 1) {  // the host splits k only with early reduce
        if (tid == 0) raise_error(S, MK_ERR_INTERNAL);
      } else if (early)
        reduce_region_finish<CT>(a.P, lds, Cfg::BN, C, a.N, r0, n0, rows, cols);
      else if (a.rs)
        rs_unit<Cfg::OCC, PT, CT>(a, r0, n0, rows, cols);
      else
        reduce_region<Cfg::OCC, PT, CT>(a.P, peers, a.n_peers, C, a.M, a.N, r0, n0, rows, cols);
      __syncthreads();
      if (tid == 0) {
        // No returned value is needed: the controller runs on compute
        // completions, the only phase in which its target matters.
        atomicAdd(xslot(S, x, X_REDUCED), 1);
        atomicAdd(xslot64(S, x, X_BUSY_R), t_busy + ticks());
        if (DYN) atomicAdd(xslot(S, x, X_STREAM), -1);
      }
    }
    __syncthreads();  // s_kind/s_tile/s_ok and LDS are reused by the next task
  }

  // ---- exit: the last workgroup out resets the claim and progress counters
  if (tid == 0) {
    if (a.tel) {  // kernel span, for telemetry only (chip-wide atomics serialise)
      atomicMin(slot64(S, S_TSTART), t_begin);
      atomicMax(slot64(S, S_TEND), ticks());
    }
    // Every counter this workgroup updated is an atomic, performed where all
    // XCDs see it; waiting for them to complete (vmcnt = 0) before counting out
    // orders them before the exit count without the agent-scope release, which
    // would write back the whole XCD L2 for every workgroup. The last workgroup
    // out acquires before it reads the counters.
    wait_stores();
    int out = __hip_atomic_fetch_add(slot32(S, S_EXIT), 1, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
    s_last = out == a.G - 1;
    if (s_last) {
      acquire_fence_agent();
      // Every tile must have been reduced unless an error stopped the kernel
      // (e.g. an XCD on which no workgroup ran would leave its queue behind).
      if (!load_relaxed(slot32(S, S_ABORT)) && sum_xcd32(S, a.n_xcd, X_REDUCED) != a.T * Cfg::RSPLIT)
        atomicCAS(slot32(S, S_ERROR), 0, MK_ERR_INTERNAL);
      if (a.tel) {
        mk_telemetry_t* t = a.tel;
        t->t_start = *slot64(S, S_TSTART);
        t->t_end = *slot64(S, S_TEND);
        t->busy_compute = sum_xcd64(S, a.n_xcd, X_BUSY_C);
        t->busy_reduce = sum_xcd64(S, a.n_xcd, X_BUSY_R);
        t->wait_reduce = sum_xcd64(S, a.n_xcd, X_WAIT_R);
        t->tiles = a.T;
        t->grid = a.G;
        t->initial_target = a.init_target;
        t->final_target = current_target(S, a.epoch, a.init_target);
        t->n_updates = *slot32(S, S_UPDATES);
        int nt = *slot32(S, S_NTRACE);
        t->n_trace = nt < MK_TRACE_CAP ? nt : MK_TRACE_CAP;
        t->role_switches = sum_xcd32(S, a.n_xcd, X_SWITCHES);
        t->reduced_by_compute = sum_xcd32(S, a.n_xcd, X_RBC) / Cfg::RSPLIT;  // units -> tiles
        t->computed_by_reducers = sum_xcd32(S, a.n_xcd, X_CBR);
        t->n_xcd = a.n_xcd;
        t->publish_ticks = sum_xcd64(S, a.n_xcd, X_PUB_T);
        t->acquire_ticks = sum_xcd64(S, a.n_xcd, X_ACQ_T);
        t->published = sum_xcd32(S, a.n_xcd, X_NPUB);
        t->acquired = sum_xcd32(S, a.n_xcd, X_NACQ);
      }
    }
  }
  // The barrier also waits for thread 0's reads above, so the reset below
  // cannot overtake them.
  __syncthreads();
  if (s_last) {
    // One word per thread: a serial loop on one thread costs over 10 us.
    for (int i = tid; i < S_COUNT; i += kThreads) {
      if (i == S_ERROR || i == S_TARGET) continue;
      __hip_atomic_store(slot64(S, i), i == S_TSTART ? ~0ull : 0ull, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ------------------------------------------------------------ AllGather+GEMM share

// "AllGather + GEMM (TP)" row of Table 3 (thelatestinai.com page): communication
// feeds compute. Every GPU's row shard of the activations is broadcast to every
// GPU, and the GEMM consumes gathered data in chunks as it arrives. One GPU's
// share: the other GPUs' shards are inputs already in HBM, and landing them in
// the gathered matrix stands in for their arrival. A band (BM rows) lands in
// column pieces (KP columns each) with one flag per piece; a tile's k-loop waits
// for each piece's flag just before it loads that piece's k-tiles, so a GEMM
// starts as soon as the first piece of its band has landed. This GPU's own bands
// are read from its shard and start at once.

// Arrival position j -> band of the gathered matrix: this GPU's own bands first,
// then the shards of ranks rank+1, rank+2, ... (mod P), each in row order.
__device__ __forceinline__ int ag_band(int j, int bps, int P, int rank) {
  const int s = (rank + j / bps) % P;
  return s * bps + j % bps;
}

// Lands piece kp of band gb: BM rows by the piece's columns, 16 bytes per lane,
// eight loads per lane in flight before their stores.
template <int BM>
__device__ __forceinline__ void ag_land(const AgArgs& a, int gb, int kp) {
  const int s = gb / a.bps;
  const int64_t r0 = (int64_t)(gb % a.bps) * BM;  // first row within the shard
  const int64_t c0 = (int64_t)kp * a.KP;
  const int64_t w = a.K - c0 < a.KP ? a.K - c0 : a.KP;  // columns (a multiple of 8)
  const uint16_t* src = s == a.rank
                            ? a.A_local + r0 * a.K + c0
                            : a.peers + ((int64_t)(s < a.rank ? s : s - 1) * a.Ms + r0) * a.K + c0;
  uint16_t* dst = a.A_full + ((int64_t)s * a.Ms + r0) * a.K + c0;
  const int cpr = (int)(w / 8);  // 16-byte chunks per row
  const int n16 = BM * cpr;
  constexpr int U = 8;
  int i = threadIdx.x;
  for (; i + (U - 1) * kThreads < n16; i += U * kThreads) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q = i + u * kThreads, r = q / cpr, c = q - r * cpr;
      v[u] = *(const u32x4*)(src + (int64_t)r * a.K + c * 8);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q = i + u * kThreads, r = q / cpr, c = q - r * cpr;
      *(u32x4*)(dst + (int64_t)r * a.K + c * 8) = v[u];
    }
  }
  for (; i < n16; i += kThreads) {
    const int r = i / cpr, c = i - r * cpr;
    *(u32x4*)(dst + (int64_t)r * a.K + c * 8) = *(const u32x4*)(src + (int64_t)r * a.K + c * 8);
  }
}

// GemmTile gate of a band that is still landing: before the loads of k-tile kt,
// every wave waits for the flag of kt's piece (once per piece). A piece is read
// only after its flag, so no cache holds a stale copy of it, provided that no
// 128-byte line holds bytes of two pieces (rows and piece widths are whole
// lines; the host checks it and otherwise sets all = 1: the first call waits
// for every piece of the band). A wait past the spin limit raises the error
// word; once the kernel is stopping no wait blocks (the tile is discarded).
struct AgGate {
  const int* flags;   // this band's piece flags
  unsigned long long* S;
  unsigned long long limit;
  int ktpp;           // 32-column k-steps per piece
  int npc;            // pieces of the band
  int all;            // 1: wait for every piece at the first k-tile
  int ready;          // pieces [0, ready] have landed
  int kmul;           // 32-column k-steps per k-tile of the GEMM
  int acq;            // 1: pieces may have landed on another XCD: acquire at agent scope
  int next_kt = 0;    // first k-tile that may need a piece beyond `ready`
  // The flag is read by a scalar load that misses the scalar cache (its count
  // is lgkmcnt), so the k-loop's direct loads in flight need not drain first, as
  // they would behind a vector load of the flag.
  __device__ __forceinline__ static int poll(const int* p) {
    int v;
    asm volatile("s_load_dword %0, %1, 0x0 glc\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
    return v;
  }
  // Every k-tile below next_kt is covered by the pieces already seen, so the
  // k-loop pays one scalar compare per k-tile; the division and the waits run
  // once per piece.
  __device__ __forceinline__ void operator()(int kt) {
    if (kt < next_kt) return;
    wait_for(kt);
  }
  __device__ __forceinline__ void wait_for(int kt) {
    // the piece that holds the k-tile's last 32 columns (a piece is a whole
    // number of k-tiles when pieces are gated one by one)
    int kp = all ? npc - 1 : (kt * kmul + kmul - 1) / ktpp;
    if (kp > npc - 1) kp = npc - 1;
    for (int p = ready + 1; p <= kp; ++p) {
      const unsigned long long w0 = ticks();
      while (poll(flags + p) == 0) {
        if (load_relaxed(slot32(S, S_ABORT))) break;
        if (ticks() - w0 > limit) {
          raise_error(S, MK_ERR_TIMEOUT);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    if (kp > ready) {
      if (acq) acquire_fence_agent();
      ready = kp;
    }
    // k-tile kt' needs piece (kt' * kmul + kmul - 1) / ktpp: beyond `ready` from
    // kt' * kmul >= (ready + 1) * ktpp - kmul + 1 on
    next_kt = all || ready >= npc - 1 ? 0x7FFFFFFF
                                      : ((ready + 1) * ktpp - kmul + 1 + kmul - 1) / kmul;
  }
};

// The fp32 tile in the accumulators, rounded to CT, into C at (m0, n0): through
// LDS (free after the GEMM's last barrier) in row-band passes, then 16-byte
// stores of whole rows.
template <class Cfg, typename CT>
__device__ __forceinline__ void store_tile_c(const GemmTile<Cfg>& g, char* lds, CT* C, int64_t M,
                                             int64_t N, int64_t m0, int64_t n0) {
  const int cols = (int)(N - n0 < Cfg::BN ? N - n0 : Cfg::BN);
  auto pass = [&](auto pass_c) {
    constexpr int PASS = decltype(pass_c)::value;
    constexpr int BAND = GemmTile<Cfg>::BAND;
    g.template stage_pass_lds<PASS>(lds);
    __syncthreads();
#pragma unroll
    for (int wm = 0; wm < 2; ++wm) {
      const int64_t r0 = m0 + wm * Cfg::WM + PASS * BAND;
      const int rows = (int)(M - r0 < BAND ? M - r0 : BAND);  // <= 0 past the edge
      copy_region_lds<CT>(lds + wm * BAND * Cfg::BN * 4, Cfg::BN, C, N, r0, n0, rows, cols);
    }
    __syncthreads();
  };
  pass(std::integral_constant<int, 0>{});
  if constexpr (GemmTile<Cfg>::NPASS > 1) pass(std::integral_constant<int, 1>{});
}

enum { AG_EXIT = 0, AG_COMPUTE = 1, AG_LAND = 2 };

// Persistent AllGather+GEMM kernel. Band j of the arrival order belongs to XCD
// j % n_xcd: the workgroups of that XCD land it and compute its tiles, so the
// landed pieces are written and read behind one L2 (the flag protocol of the
// tile flags). Each XCD has a tile queue (its bands in arrival order, every
// tile column of a band before the next band) and a landing queue (piece 0 of
// each of its other-GPU bands, then piece 1 of each, ..., then its own bands'
// pieces, which the gathered matrix holds too). The first workgroups to arrive
// on an XCD (its share of n_comm) only land pieces while any are left, and
// never wait. A workgroup holding a tile of a landing band first lands pieces
// while the band's first piece has not landed and pieces are unclaimed (and,
// on an XCD without landing workgroups, until every piece of the band is
// claimed); then it runs the GEMM, whose gate waits for each later piece. Every
// piece it can wait for is claimed by a workgroup that lands it without
// waiting, so no wait can stall the kernel.
template <class Cfg, typename CT>
__global__ __launch_bounds__(kThreads, Cfg::OCC) void ag_kernel(AgArgs a) {
  __shared__ __align__(1024) char lds[Cfg::LDS_BYTES];
  __shared__ int s_kind, s_idx, s_last;
  const int tid = threadIdx.x;
  unsigned long long* S = a.slots;
  const int hw_xcd = xcc_id();
  const int x = hw_xcd % a.n_xcd;
  // This XCD's bands: arrival positions x + i*n_xcd for i < nb; the first nl are
  // this GPU's own, the other nbp are landing.
  const int nb = a.NB > x ? (a.NB - x + a.n_xcd - 1) / a.n_xcd : 0;
  const int nl = a.bps > x ? (a.bps - x + a.n_xcd - 1) / a.n_xcd : 0;
  const int nbp = nb - nl;
  const int cnt = nb * a.tiles_n;
  const int units = nb * a.npc;
  const int tx = a.n_comm / a.n_xcd + (x < a.n_comm % a.n_xcd ? 1 : 0);
  int* cnext = xslot(S, x, X_COMPUTE_NEXT);
  int* lnext = xslot(S, x, X_REDUCE_NEXT);
  int rank = -1, held = -1;  // thread 0: arrival rank; a claimed tile of a landing band
  unsigned long long w0 = 0;

  for (;;) {
    if (tid == 0) {
      int kind = AG_EXIT, idx = -1;
      for (;;) {
        const int abort = load_relaxed(slot32(S, S_ABORT));
        const int cn = load_relaxed(cnext);
        const int ln = load_relaxed(lnext);
        if (rank < 0) {
          rank = atomicAdd(xslot(S, x, X_ARRIVE), 1);
          if (a.flag_scope == 0 && !same_xcd_queue(S, x, hw_xcd)) break;
        }
        if (abort) break;
        if (rank < tx && ln < units) {  // a landing workgroup while pieces are left
          const int u = atomicAdd(lnext, 1);
          if (u < units) {
            kind = AG_LAND;
            idx = u;
            break;
          }
          continue;
        }
        if (held >= 0) {
          const int i = held / a.tiles_n - nl;  // position among the landing bands
          const int gb = ag_band(x + (held / a.tiles_n) * a.n_xcd, a.bps, a.P, a.rank);
          const bool first = a.npc == 0 || load_relaxed(a.landed + gb * kAgMaxPieces) != 0;
          // unit of the band's last piece: all pieces claimed once the queue is past it
          const bool claimed = ln > (a.npc - 1) * nbp + i;
          if ((!first || (tx == 0 && !claimed)) && ln < units) {
            const int u = atomicAdd(lnext, 1);  // land a piece rather than wait
            if (u < units) {
              kind = AG_LAND;
              idx = u;
              w0 = 0;
              break;
            }
          }
          if (first) {
            kind = AG_COMPUTE;
            idx = held;
            held = -1;
            break;
          }
          if (w0 == 0) w0 = ticks();  // the first piece is claimed: wait for it
          if (ticks() - w0 > a.spin_limit) {
            raise_error(S, MK_ERR_TIMEOUT);
            break;
          }
          backoff_sleep(1);
          continue;
        }
        if (cn < cnt) {
          const int t = atomicAdd(cnext, 1);
          if (t < cnt) {
            if (t / a.tiles_n < nl) {  // a band of this GPU's own shard
              kind = AG_COMPUTE;
              idx = t;
              break;
            }
            held = t;
            w0 = 0;
            continue;
          }
        }
        if (ln < units) {
          const int u = atomicAdd(lnext, 1);
          if (u < units) {
            kind = AG_LAND;
            idx = u;
          }
        }
        break;
      }
      s_kind = kind;
      s_idx = idx;
    }
    __syncthreads();
    const int kind = s_kind, idx = s_idx;
    if (kind == AG_EXIT) break;
    if (kind == AG_LAND) {
      int i, kp;
      if (idx < nbp * a.npc) {  // other GPUs' bands, piece-major
        kp = idx / nbp;
        i = nl + idx % nbp;
      } else {                  // this GPU's own bands
        const int v = idx - nbp * a.npc;
        kp = v / nl;
        i = v % nl;
      }
      const int gb = ag_band(x + i * a.n_xcd, a.bps, a.P, a.rank);
      ag_land<Cfg::BM>(a, gb, kp);
      wait_stores();    // this wave's stores have reached the L2
      __syncthreads();  // ... and every other wave's
      if (tid == 0) {
        if (a.flag_scope == 0) store_flag(a.landed + gb * kAgMaxPieces + kp, 1);
        else publish_flag_agent(a.landed + gb * kAgMaxPieces + kp, 1);
        atomicAdd(xslot(S, x, X_REDUCED), 1);
      }
    } else {
      const int pos = idx / a.tiles_n, tn = idx % a.tiles_n;
      const int gb = ag_band(x + pos * a.n_xcd, a.bps, a.P, a.rank);
      const int sh = gb / a.bps;
      const int64_t rs = (int64_t)(gb % a.bps) * Cfg::BM;  // first row within the shard
      const int64_t m0 = (int64_t)sh * a.Ms + rs, n0 = (int64_t)tn * Cfg::BN;
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no load of the last task in flight
      GemmTile<Cfg> g;
      if (sh == a.rank) {
        g.run(a.A_local, a.B, a.Ms, a.N, a.K, rs, n0, lds);
      } else {
        AgGate gate{a.landed + gb * kAgMaxPieces, S, a.spin_limit, a.ktpp, a.npc, !a.inloop, -1,
                    Cfg::BK / 32, a.flag_scope};
        g.run(a.A_full, a.B, a.M, a.N, a.K, m0, n0, lds, gate);
      }
      store_tile_c<Cfg, CT>(g, lds, (CT*)a.C, a.M, a.N, m0, n0);
      if (tid == 0) atomicAdd(xslot(S, x, X_COMPUTED), 1);
    }
    __syncthreads();  // s_kind/s_idx and LDS are reused by the next task
  }

  // ---- exit: the last workgroup out checks the work and resets the counters
  if (tid == 0) {
    wait_stores();
    int out = __hip_atomic_fetch_add(slot32(S, S_EXIT), 1, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
    s_last = out == a.G - 1;
    if (s_last) {
      acquire_fence_agent();
      if (!load_relaxed(slot32(S, S_ABORT)) &&
          (sum_xcd32(S, a.n_xcd, X_COMPUTED) != a.T ||
           sum_xcd32(S, a.n_xcd, X_REDUCED) != a.NB * a.npc))
        atomicCAS(slot32(S, S_ERROR), 0, MK_ERR_INTERNAL);
    }
  }
  __syncthreads();
  if (s_last) {
    for (int i = tid; i < S_COUNT; i += kThreads) {
      if (i == S_ERROR || i == S_TARGET) continue;
      __hip_atomic_store(slot64(S, i), i == S_TSTART ? ~0ull : 0ull, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
    for (int i = tid; i < a.NB * kAgMaxPieces; i += kThreads)
      __hip_atomic_store(a.landed + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ------------------------------------------------------------ flag hand-off microbenchmark

// Scopes: 0 = stores complete + relaxed flag, workgroup-scope invalidate (shown
// not to carry data); 1 = agent-scope release and acquire; 2 = the fused
// kernel's protocol: stores complete + relaxed flag, agent-scope acquire.
// Two workgroups hand a flag back and forth `iters` times: side 0 writes a data
// word (plain store), publishes step i (the tile flag's publish: stores
// complete, then the flag store) and waits for side 1 to publish it back; side 1
// waits for step i (poll, then the consumer's cache maintenance), reads the data
// word with a plain load and counts values other than step i (a message-passing
// litmus: a stale read means the protocol does not carry data). One hand-off is
// the path of a tile from its compute workgroup to its reducer. Side 1 is
// workgroup n_xcd (dealt to the XCD of workgroup 0) or, with cross_xcd,
// workgroup 1 (the next XCD). Every wait is bounded: a side that times out
// records it and leaves, and so does the other side at its own limit.
// out: [0] ticks of the whole exchange (side 0), [1] 1 if a wait timed out,
// [2], [3] the XCDs of side 0 and side 1, [4] stale data reads (side 1).
__global__ void pingpong_kernel(unsigned long long* S, unsigned call, int iters, int scope,
                                unsigned long long limit, unsigned long long* out, int side1) {
  const int b = blockIdx.x;
  if ((b != 0 && b != side1) || threadIdx.x != 0) return;
  const int me = b == 0 ? 0 : 1;
  unsigned long long* mine = slot64(S, me == 0 ? S_PING : S_PONG);
  unsigned long long* theirs = slot64(S, me == 0 ? S_PONG : S_PING);
  unsigned long long* payload = slot64(S, S_PAYLOAD);
  out[2 + me] = (unsigned long long)xcc_id();
  const unsigned long long base = (unsigned long long)call << 32;
  const unsigned long long t0 = ticks();
  int timed_out = 0;
  unsigned long long stale = 0;
  for (int i = 1; i <= iters && !timed_out; ++i) {
    const unsigned long long want = base | (unsigned)i;
    if (me == 1) {  // wait for side 0's step i, then read what it carries
      const unsigned long long w0 = ticks();
      while (__hip_atomic_load(theirs, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != want) {
        if (ticks() - w0 > limit) { timed_out = 1; break; }
      }
      if (scope == 0) inv_group_scope();
      else acquire_fence_agent();  // scopes 1 and 2
      if (!timed_out && *payload != want) ++stale;
    } else {
      *payload = want;
    }
    if (!timed_out) {  // publish step i
      wait_stores();
      if (scope != 1) __hip_atomic_store(mine, want, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else __hip_atomic_store(mine, want, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (me == 0 && !timed_out) {  // wait for side 1 to hand step i back
      const unsigned long long w0 = ticks();
      while (__hip_atomic_load(theirs, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != want) {
        if (ticks() - w0 > limit) { timed_out = 1; break; }
      }
      if (scope == 0) inv_group_scope();
      else acquire_fence_agent();
    }
  }
  if (me == 0) out[0] = ticks() - t0;
  else out[4] = stale;
  if (timed_out) out[1] = 1;
}

// Baseline AllGather: every shard into the gathered matrix, 16 bytes per lane.
__global__ __launch_bounds__(kThreads) void ag_copy_kernel(AgCopyArgs a) {
  const int64_t per = a.Ms * a.K / 8;  // 16-byte chunks per shard
  const int64_t total = per * a.P;
  const int64_t step = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total; i += step) {
    const int s = (int)(i / per);
    const int64_t o = i - (int64_t)s * per;
    const uint16_t* src =
        s == a.rank ? a.A_local : a.peers + (int64_t)(s < a.rank ? s : s - 1) * a.Ms * a.K;
    ((u32x4*)a.A_full)[i] = ((const u32x4*)src)[o];
  }
}

// Baseline GEMM writing C in its own type (one workgroup per tile, the tile map
// of gemm_kernel).
template <class Cfg, typename CT>
__global__ __launch_bounds__(kThreads, 1) void gemm_c_kernel(GemmArgs a, CT* C) {
  __shared__ __align__(1024) char lds[Cfg::LDS_BYTES];
  const int T = a.tiles_m * a.tiles_n;
  const int b = blockIdx.x;
  int t = b;
  if (a.n_xcd > 1 && T % a.n_xcd == 0) t = (b % a.n_xcd) * (T / a.n_xcd) + b / a.n_xcd;
  int tm, tn;
  fused_tile_coords(t, a.tiles_m, a.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * Cfg::BM, n0 = (int64_t)tn * Cfg::BN;
  GemmTile<Cfg> g;
  g.run(a.A, a.B, a.M, a.N, a.K, m0, n0, lds);
  store_tile_c<Cfg, CT>(g, lds, C, a.M, a.N, m0, n0);
}

// ------------------------------------------------------------ baseline kernels

template <class Cfg>
__global__ __launch_bounds__(Cfg::NW * 64, 1) void gemm_kernel(GemmArgs a) {
  __shared__ __align__(1024) char lds[Cfg::LDS_BYTES];
  // The dispatcher deals workgroups to XCDs in turn (workgroup b on XCD
  // b % n_xcd). Giving each XCD a contiguous range of the tile order, mapped as
  // in the fused kernel, lets the tiles that run together on an XCD share A and B
  // panels in its L2 (dealt in turn, each XCD would read every B panel).
  const int T = a.tiles_m * a.tiles_n;
  const int b = blockIdx.x;
  int t = b;
  if (a.n_xcd > 1 && T % a.n_xcd == 0) t = (b % a.n_xcd) * (T / a.n_xcd) + b / a.n_xcd;
  int tm, tn;
  fused_tile_coords(t, a.tiles_m, a.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * Cfg::BM, n0 = (int64_t)tn * Cfg::BN;
  GemmTile<Cfg> g;
  g.run(a.A, a.B, a.M, a.N, a.K, m0, n0, lds);
  g.store_partial(a.P, a.M, a.N, m0, n0);
}

// Ring depth of the grid-stride reduce: one chunk in flight while one is summed
// once a chunk holds 9 or more 16-byte loads (measured on MI355X: 7 bfloat16
// peers 197 us with depth 2 against 217 us with depth 3 on 8192 x 8192, 15 peers
// 855 against 967 us on 16384 x 8192), the in-place reducers' depth below that.
template <typename PT, int NP>
__host__ __device__ constexpr int span_ring_depth() {
  constexpr int loads = 2 + NP * (sizeof(PT) == 2 ? 1 : 2);
  return loads >= 9 ? 2 : ring_depth<1, PT, NP>();
}

// Chunks of 8 elements [0, total) of a dense span, thread t of the grid taking
// t, t + stride, ...; the same sum, in the same order, as every other path.
// Peer counts with a compile-time ring keep the next chunk's loads in flight
// while one is summed; the others fetch a batch of peers at a time.
template <typename PT, typename CT>
__device__ __forceinline__ void reduce_span(const float* __restrict__ P, const PT* __restrict__ peers,
                                            int n_peers, int64_t peer_stride, CT* __restrict__ C,
                                            int total, int t, int stride) {
  // the span as one row of `total` chunks (row pitch 8 * total)
  const int64_t pitch = (int64_t)total * 8;
#define MK_SPAN_RING(NPV)                                                                 \
  case NPV:                                                                               \
    if constexpr (ring_fits<1, PT, NPV>()) {                                              \
      const PT* pr[NPV];                                                                  \
      _Pragma("unroll") for (int s = 0; s < NPV; ++s) pr[s] = peers + s * peer_stride;    \
      typedef SumOp<PT, NPV, PartialGlobal, OutC<CT>> Op;                                 \
      ReduceRing<span_ring_depth<PT, NPV>(), Op>::run_strided(                           \
          Op{PartialGlobal{P}, pr, OutC<CT>{C}}, total, total, pitch, pitch, t, stride);  \
      return;                                                                             \
    }                                                                                     \
    break;
  switch (n_peers) {
    MK_RING_PEER_COUNTS(MK_SPAN_RING)
    default: break;
  }
#undef MK_SPAN_RING
  int64_t q = t;
  for (; q + stride < total; q += 2 * (int64_t)stride) {
    int64_t e[2] = {q * 8, (q + stride) * 8};
    reduce_chunks<2, PT, CT>(P, peers, n_peers, peer_stride, C, e);
  }
  if (q < total) {
    int64_t e[1] = {q * 8};
    reduce_chunks<1, PT, CT>(P, peers, n_peers, peer_stride, C, e);
  }
}

// The two-kernel baseline's reduce (and the per-chunk reduce of the two-stream
// schedule): C = round(peers' sum + P) over a dense M x N region, one
// workgroup per compute unit walking the region grid-stride. The region is
// taken in bands of whole rows of at most 2^29 elements, so that every byte
// offset from a band's first element fits in 32 bits (N <= 2^22 is checked on
// the host).
template <typename PT, typename CT>
__global__ __launch_bounds__(kThreads) void reduce_kernel(ReduceArgs a) {
  const PT* peers = (const PT*)a.peers;
  CT* C = (CT*)a.C;
  const int t = (int)(blockIdx.x * kThreads + threadIdx.x);
  const int stride = (int)(gridDim.x * kThreads);
  const int64_t band = ((int64_t)1 << 29) / a.N;
  for (int64_t m0 = 0; m0 < a.M; m0 += band) {
    const int64_t rows = a.M - m0 < band ? a.M - m0 : band;
    const int64_t e0 = m0 * a.N;
    reduce_span<PT, CT>(a.P + e0, peers + e0, a.n_peers, a.peer_stride, C + e0,
                        (int)(rows * a.N / 8), t, stride);
  }
}

// Workspace of mk_gemm_ar_local_noalloc: every GPU the library runs on holds
// its own copy of this array until the process ends. Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the symbol):
// it looks up each device's address with hipGetSymbolAddress and passes that.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t noalloc_scratch_address(void** p) {
  return hipGetSymbolAddress(p, HIP_SYMBOL(scratch));
}

// Workspace initialisation: flags to 0, slots to their reset values.
__global__ void ws_init_kernel(int* flags, int n_flags, unsigned long long* slots) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n_flags; i += gridDim.x * blockDim.x)
    flags[i] = 0;
  if (slots && blockIdx.x == 0) {
    for (int i = threadIdx.x; i < S_COUNT * kSlotWords; i += blockDim.x)
      slots[i] = (i == S_TSTART * kSlotWords) ? ~0ull : 0ull;
  }
}

// Clears the error word only (after the host has read it).
__global__ void clear_error_kernel(unsigned long long* slots) {
  if (threadIdx.x == 0) slots[(size_t)S_ERROR * kSlotWords] = 0ull;
}

// ------------------------------------------------------------ matrix-core peak

// Matrix-core ceiling of the chip: every wave issues `iters` rounds of eight
// independent v_mfma_f32_32x32x16_bf16 on register operands (no memory traffic
// in the loop), then each lane stores the sum of its accumulators so that no
// product is dead. 32768 flops per MFMA.
__global__ __launch_bounds__(kThreads, 1) void mfma_peak_kernel(int iters, float* out) {
  const int tid = threadIdx.x;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(float)((tid + i) & 7);
    b[i] = (__bf16)(float)((tid * 3 + i) & 7);
  }
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[j][i] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += acc[j][i];
  out[(size_t)blockIdx.x * kThreads + tid] = sum;
}

// ------------------------------------------------------------ wave-specialised AllReduce

// Persistent fused GEMM+AllReduce in which the GEMM and the reduce overlap inside
// each workgroup: one workgroup per compute unit. Waves 0-3 run the GEMM of the
// workgroup's tiles one after another (the fp32 accumulators in their
// registers); the streaming waves (two or four, ws_stream) meanwhile reduce the
// tile before: its partial
// waits in LDS, where the GEMM waves staged it when their k-loop ended, and the
// streaming waves add it to the sum of the peers' slices and write C. The
// matrix cores thus work while the peers stream from HBM, and no partial goes
// through device memory. With 64x256 tiles two streaming waves streamed as fast
// as four or eight on MI355X (16384x8192x512 with 15 peers: 817, 817 and 838 us)
// and left more of each CU's memory pipeline to the GEMM's loads; deeper rings
// were slower (859 us). 32-deep k-tiles there (64-deep ones measured slower).
//
// Two tile shapes, each with its fp32 partial (64 KiB) and its k-stages in the
// LDS: 64 x 256, whose rows are 512 contiguous bytes of every bfloat16 peer (the
// 256-byte pieces of 128 x 128 tiles streamed about 15% slower from HBM on
// MI355X), for shapes where the stream dominates; 128 x 128, which load fewer A
// and B bytes per output, where the GEMM weighs more. Tiles are dealt
// statically: XCD x owns a contiguous range of the tile order, served by its
// workgroups in turn.
//
// Both groups pass the same workgroup barriers in each round: the GEMM's k-loop
// holds one per k-tile and a last one after it; the streaming waves spread as
// many as the k-loop has over their chunks and meet the last one when their
// reads of the partial are done. After that barrier the GEMM waves stage the new
// partial, and one more barrier hands it over. The round after the last GEMM
// only streams.
using TWs = TileCfg<64, 256>;     // 320 rows and columns of A and B per 16 K outputs
// 256 per 16 K outputs; 64-deep k-tiles in three stages, which with the 64 KiB
// partial fill the 160 KiB of LDS (mlp 284-285 us against 292-296 us with 32-deep
// k-tiles in four stages, and 3-9% faster on every shape of the rule's table)
using TWs128 = TileCfg<128, 128, 64, 3>;
// Streaming threads per workgroup (STREAM): two waves, or four beside the
// 128x128 GEMM when each streaming lane has one chunk in flight (ring depth 2:
// 15 bfloat16 peers, say; the host's ws_wide). Measured on MI355X, same
// machine: 16384x8192x512 with 15 peers (64x256 tiles) 807-810 us with two
// waves, 891-893 with three, 818-821 with four; 4096x8192x1792 with 15 peers
// (128x128) 282-284 us with two, 285-287 with three, 276 with four; 8192x8192x
// 1024 with 7 peers (128x128, three chunks in flight) 291 us with two, 314 with
// four.
template <class Cfg, typename PT, typename CT, int STREAM>
__global__ __launch_bounds__(kThreads + STREAM, 1) void ws_kernel(FusedArgs a) {
  constexpr int kWsStream = STREAM;
  static_assert(GemmTile<Cfg>::NPASS == 1, "the whole fp32 tile is staged in one pass");
  __shared__ __align__(1024) char lds[Cfg::LDS_BYTES + Cfg::BM * Cfg::BN * 4];
  char* const part = lds + Cfg::LDS_BYTES;
  const int b = blockIdx.x, G = gridDim.x;
  // this workgroup's tiles: q0 + s, q0 + s + per, ... below q1
  int q0 = 0, q1 = a.T, s = b, per = G;
  if (a.n_xcd > 1 && G % a.n_xcd == 0) {
    const int x = b % a.n_xcd;  // workgroups are dealt to the XCDs in turn
    q0 = (int)(((int64_t)x * a.T) / a.n_xcd);
    q1 = (int)(((int64_t)(x + 1) * a.T) / a.n_xcd);
    s = b / a.n_xcd;
    per = G / a.n_xcd;
  }
  const int n_my = q1 - q0 > s ? (q1 - q0 - s + per - 1) / per : 0;
  const int KT = (int)((a.K + Cfg::BK - 1) / Cfg::BK);
  auto origin = [&](int j, int64_t& m0, int64_t& n0) {
    int tm, tn;
    // row groups of 1024 output rows whatever the tile height (16 rows of 64x256
    // tiles: 805 against 815 us on 16384x8192x512 with 15 peers; 8 rows of
    // 128x128 tiles: 293 against 302 us on 4096x8192x1792 with 16 rows)
    fused_tile_coords<1024 / Cfg::BM>(q0 + s + j * per, a.tiles_m, a.tiles_n, tm, tn);
    m0 = (int64_t)tm * Cfg::BM;
    n0 = (int64_t)tn * Cfg::BN;
  };
  // Each group runs its own loop over the rounds (what one keeps in registers
  // across rounds is not live in the other's code).
  if (threadIdx.x < kThreads) {
    for (int j = 0; j <= n_my; ++j) {
      if (j < n_my) {
        int64_t m0, n0;
        origin(j, m0, n0);
        GemmTile<Cfg> g;
        g.run(a.A, a.B, a.M, a.N, a.K, m0, n0, lds);  // KT + 1 barriers (none when K = 0)
        if (KT == 0) __syncthreads();
        g.template stage_pass_lds<0>(part);
      } else {
        __syncthreads();  // stands for the k-loop's last barrier
      }
      __syncthreads();  // the new partial is staged
    }
  } else {
    const PT* peers = (const PT*)a.peers;
    CT* C = (CT*)a.C;
    const int t = threadIdx.x - kThreads;
    for (int j = 0; j <= n_my; ++j) {
      // barriers of this round's k-loop before its last one
      const int nb = j < n_my ? KT : 0;
      if (j > 0) {
        int64_t m0, n0;  // the tile whose partial is staged
        origin(j - 1, m0, n0);
        const int rows = (int)(a.M - m0 < Cfg::BM ? a.M - m0 : Cfg::BM);
        const int cols = (int)(a.N - n0 < Cfg::BN ? a.N - n0 : Cfg::BN);
        // a peer count without a ring is never launched here (the host checks);
        // were it, C would be left unwritten: report it
        if (!stream_region_lds<kWsStream, PT, CT>(part, Cfg::BN, peers, a.n_peers, C, a.M, a.N,
                                                  m0, n0, rows, cols, t, nb) &&
            t == 0)
          atomicCAS(slot32(a.slots, S_ERROR), 0, MK_ERR_INTERNAL);  // (no abort: nothing waits)
      } else {
        for (int i = 0; i < nb; ++i) __syncthreads();
      }
      __syncthreads();  // the k-loop's last barrier: the staged partial is consumed
      __syncthreads();  // the new partial is staged
    }
  }
}

// Every tile reduced in place by the workgroup that computes it, the tiles
// dealt in a fixed order: XCD x owns a contiguous range of the tile order
// (fused_tile_coords), served by its workgroups in turn, as the per-XCD queues
// of fused_kernel serve it, but without claims, flags, counters or a
// controller, so the kernel keeps only the GEMM's and the reduce's state in
// registers (on MI355X, 8192^3 with 7 peers: 1087-1096 us against 1113-1121 us
// for the claim-queue kernel in the same run).
template <class Cfg, typename PT, typename CT>
__global__ __launch_bounds__(Cfg::NW * 64, 1) void inplace_kernel(FusedArgs a) {
  __shared__ __align__(1024) char lds[Cfg::LDS_BYTES];
  const int b = blockIdx.x, G = gridDim.x;
  int q0 = 0, q1 = a.T, s = b, per = G;
  if (a.n_xcd > 1 && G % a.n_xcd == 0) {
    const int x = b % a.n_xcd;  // workgroups are dealt to the XCDs in turn
    q0 = (int)(((int64_t)x * a.T) / a.n_xcd);
    q1 = (int)(((int64_t)(x + 1) * a.T) / a.n_xcd);
    s = b / a.n_xcd;
    per = G / a.n_xcd;
  }
  const PT* peers = (const PT*)a.peers;
  CT* C = (CT*)a.C;
  for (int q = q0 + s; q < q1; q += per) {
    int tm, tn;
    fused_tile_coords(q, a.tiles_m, a.tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * Cfg::BM, n0 = (int64_t)tn * Cfg::BN;
    GemmTile<Cfg> g;
    g.run(a.A, a.B, a.M, a.N, a.K, m0, n0, lds);
    inplace_tile<Cfg, PT, CT>(g, lds, peers, a.n_peers, C, a.M, a.N, m0, n0);
  }
}

// ------------------------------------------------------------ host-side launchers

using T256 = TileCfg<256, 256, 64, 2>;  // 64-deep k-tiles, two LDS stages
// The same tile computed by eight waves in a 2 x 4 grid (128 x 64 each, two
// waves per SIMD) for the in-place kernel: bitwise the same products; on MI355X
// 8192^3 ran 895-900 us against 919-951 us with four waves (GEMM alone), and the
// fused call on 8192^3 with 7 peers 1024-1028 us against 1039-1045 us.
using T256w8 = TileCfg<256, 256, 64, 2, 8, 4>;
using T128 = TileCfg<128, 128>;
// Few-tile shapes: every tile reduced in place; 64-deep k-tiles in four stages
// (eight stages measured slower on the 128x8192x1792 shard: 31.9 against 30.0 us).
using T64 = TileCfg<64, 64, 64, 4>;

template <class Cfg, bool DYN>
static const void* fused_ptr(int pt, int ct) {
  if (pt == MK_DT_BF16 && ct == MK_DT_BF16)
    return (const void*)fused_kernel<Cfg, uint16_t, uint16_t, DYN>;
  if (pt == MK_DT_BF16 && ct == MK_DT_F32) return (const void*)fused_kernel<Cfg, uint16_t, float, DYN>;
  if (pt == MK_DT_F32 && ct == MK_DT_BF16) return (const void*)fused_kernel<Cfg, float, uint16_t, DYN>;
  return (const void*)fused_kernel<Cfg, float, float, DYN>;
}

template <class Cfg, int STREAM>
static const void* ws_ptr(int pt, int ct) {
  if (pt == MK_DT_BF16 && ct == MK_DT_BF16) return (const void*)ws_kernel<Cfg, uint16_t, uint16_t, STREAM>;
  if (pt == MK_DT_BF16 && ct == MK_DT_F32) return (const void*)ws_kernel<Cfg, uint16_t, float, STREAM>;
  if (pt == MK_DT_F32 && ct == MK_DT_BF16) return (const void*)ws_kernel<Cfg, float, uint16_t, STREAM>;
  return (const void*)ws_kernel<Cfg, float, float, STREAM>;
}

template <class Cfg>
static const void* inplace_ptr(int pt, int ct) {
  if (pt == MK_DT_BF16 && ct == MK_DT_BF16) return (const void*)inplace_kernel<Cfg, uint16_t, uint16_t>;
  if (pt == MK_DT_BF16 && ct == MK_DT_F32) return (const void*)inplace_kernel<Cfg, uint16_t, float>;
  if (pt == MK_DT_F32 && ct == MK_DT_BF16) return (const void*)inplace_kernel<Cfg, float, uint16_t>;
  return (const void*)inplace_kernel<Cfg, float, float>;
}

const void* fused_kernel_ptr(int shape, int pt, int ct, int variant) {
  const int dyn = variant;
  if (shape == SHAPE_WS) return ws_ptr<TWs, 128>(pt, ct);
  if (shape == SHAPE_WS128) return variant ? ws_ptr<TWs128, 256>(pt, ct) : ws_ptr<TWs128, 128>(pt, ct);
  if (shape == SHAPE_64) return fused_ptr<T64, false>(pt, ct);  // no dynamic variant
  if (dyn) return shape == SHAPE_256 ? fused_ptr<T256, true>(pt, ct) : fused_ptr<T128, true>(pt, ct);
  return shape == SHAPE_256 ? fused_ptr<T256, false>(pt, ct) : fused_ptr<T128, false>(pt, ct);
}

hipError_t launch_mfma_peak(int iters, int grid, float* out, hipStream_t s) {
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(grid), dim3(kThreads), 0, s, iters, out);
  return hipGetLastError();
}

const void* ag_kernel_ptr(int shape, int ct) {
  if (shape == SHAPE_256)
    return ct == MK_DT_BF16 ? (const void*)ag_kernel<T256, uint16_t> : (const void*)ag_kernel<T256, float>;
  return ct == MK_DT_BF16 ? (const void*)ag_kernel<T128, uint16_t> : (const void*)ag_kernel<T128, float>;
}

const void* gemm_kernel_ptr(int shape, int waves8) {
  if (shape == SHAPE_64) return (const void*)gemm_kernel<T64>;
  if (shape == SHAPE_256 && waves8) return (const void*)gemm_kernel<T256w8>;
  return shape == SHAPE_256 ? (const void*)gemm_kernel<T256> : (const void*)gemm_kernel<T128>;
}

const void* reduce_kernel_ptr(int pt, int ct) {
  if (pt == MK_DT_BF16 && ct == MK_DT_BF16) return (const void*)reduce_kernel<uint16_t, uint16_t>;
  if (pt == MK_DT_BF16 && ct == MK_DT_F32) return (const void*)reduce_kernel<uint16_t, float>;
  if (pt == MK_DT_F32 && ct == MK_DT_BF16) return (const void*)reduce_kernel<float, uint16_t>;
  return (const void*)reduce_kernel<float, float>;
}

int shape_threads(int shape, int variant) {
  if (shape == SHAPE_WS) return kThreads + 128;
  if (shape == SHAPE_WS128) return kThreads + (variant ? 256 : 128);
  return kThreads;
}
int shape_bm(int shape) {
  if (shape == SHAPE_WS) return TWs::BM;
  if (shape == SHAPE_WS128) return TWs128::BM;
  return shape == SHAPE_256 ? 256 : (shape == SHAPE_64 ? 64 : 128);
}
int shape_bn(int shape) {
  if (shape == SHAPE_WS) return TWs::BN;
  if (shape == SHAPE_WS128) return TWs128::BN;
  return shape == SHAPE_256 ? 256 : (shape == SHAPE_64 ? 64 : 128);
}

hipError_t launch_ws_init(int* flags, int n_flags, unsigned long long* slots, hipStream_t s) {
  hipLaunchKernelGGL(ws_init_kernel, dim3(64), dim3(256), 0, s, flags, n_flags, slots);
  return hipGetLastError();
}

hipError_t launch_clear_error(unsigned long long* slots, hipStream_t s) {
  hipLaunchKernelGGL(clear_error_kernel, dim3(1), dim3(64), 0, s, slots);
  return hipGetLastError();
}

hipError_t launch_fused(int shape, int pt, int ct, const FusedArgs& a, hipStream_t s) {
  // the host sets static_tiles for 256x256 tiles only
  const int variant = is_ws(shape) ? a.ws_wide : a.dyn;
  if (a.static_tiles && shape == SHAPE_256) {
    const void* f = a.waves8 ? inplace_ptr<T256w8>(pt, ct) : inplace_ptr<T256>(pt, ct);
    void* args[] = {(void*)&a};
    return hipLaunchKernel(f, dim3(a.G), dim3(a.waves8 ? 512 : kThreads), args, 0, s);
  }
  const void* f = fused_kernel_ptr(shape, pt, ct, variant);
  void* args[] = {(void*)&a};
  return hipLaunchKernel(f, dim3(a.G), dim3(shape_threads(shape, variant)), args, 0, s);
}

hipError_t launch_gemm(int shape, const GemmArgs& a, hipStream_t s) {
  const bool w8 = shape == SHAPE_256 && a.waves8;
  const void* f = gemm_kernel_ptr(shape, w8);
  void* args[] = {(void*)&a};
  return hipLaunchKernel(f, dim3(a.tiles_m * a.tiles_n), dim3(w8 ? 512 : kThreads), args, 0, s);
}

hipError_t launch_reduce(int pt, int ct, const ReduceArgs& a, int grid, hipStream_t s) {
  const void* f = reduce_kernel_ptr(pt, ct);
  void* args[] = {(void*)&a};
  return hipLaunchKernel(f, dim3(grid), dim3(kThreads), args, 0, s);
}

hipError_t launch_ag(int shape, int ct, const AgArgs& a, hipStream_t s) {
  const void* f = ag_kernel_ptr(shape, ct);
  void* args[] = {(void*)&a};
  return hipLaunchKernel(f, dim3(a.G), dim3(kThreads), args, 0, s);
}

hipError_t launch_ag_copy(const AgCopyArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL(ag_copy_kernel, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm_c(int shape, int ct, const GemmArgs& a, void* C, hipStream_t s) {
  const int T = a.tiles_m * a.tiles_n;
  if (shape == SHAPE_256) {
    if (ct == MK_DT_BF16)
      hipLaunchKernelGGL((gemm_c_kernel<T256, uint16_t>), dim3(T), dim3(kThreads), 0, s, a, (uint16_t*)C);
    else
      hipLaunchKernelGGL((gemm_c_kernel<T256, float>), dim3(T), dim3(kThreads), 0, s, a, (float*)C);
  } else {
    if (ct == MK_DT_BF16)
      hipLaunchKernelGGL((gemm_c_kernel<T128, uint16_t>), dim3(T), dim3(kThreads), 0, s, a, (uint16_t*)C);
    else
      hipLaunchKernelGGL((gemm_c_kernel<T128, float>), dim3(T), dim3(kThreads), 0, s, a, (float*)C);
  }
  return hipGetLastError();
}

hipError_t launch_pingpong(unsigned long long* slots, unsigned call, int iters, int scope,
                           int cross_xcd, unsigned long long limit, unsigned long long* out,
                           hipStream_t s) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int n_xcd = cus / 32 > 1 ? cus / 32 : 1;
  // workgroup n_xcd is dealt to the XCD of workgroup 0, workgroup 1 to the next
  const int side1 = cross_xcd || n_xcd == 1 ? 1 : n_xcd;
  hipLaunchKernelGGL(pingpong_kernel, dim3(side1 + 1), dim3(64), 0, s, slots, call, iters, scope,
                     limit, out, side1);
  return hipGetLastError();
}

}  // namespace mk
