// mk_api.cpp -- host side of libmk.so: argument validation, per-(device,
// stream) workspaces, kernel selection and launch. See include/mk.h for the
// contract of each entry point.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <vector>
#include <string>
#include <utility>

#include "mk.h"
#include "mk_controller.h"
#include "mk_kernels.h"

namespace {

thread_local std::string g_last_error;

mk_status_t fail(mk_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

mk_status_t hip_fail(hipError_t e, const char* what) {
  return fail(MK_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ------------------------------------------------------------ options

struct Options {
  int64_t spin_timeout_us = 2000000;
  int64_t withhold_tile = -1;
  int64_t ctrl_period = 8;
  int64_t tile_shape = mk::SHAPE_AUTO;
  int64_t flag_scope = 0;
  int64_t reducer_cap = 0;  // 0: derived from HBM bandwidth and a reducer's streaming rate
  int64_t inplace = -1;     // -1: automatic; 0: none; n: the last n tiles of each XCD's queue
  int64_t early = -1;       // reducers sum a unit's peers before its tile is finished: -1 auto
  int64_t ksplit = -1;      // early-reduce tiles computed as two k-halves: -1 auto, 1 off, 2 on
  int64_t stream_cu_split = 0;  // two-stream schedule: compute units of the reduce stream (0: no masks)
  int64_t static_tiles = 2;  // all-in-place 256x256 tiles: 2 the in-place kernel with eight waves
                             // where its rings fit, 1 with four, 0 claim queues
};
std::mutex g_opt_mu;
Options g_opt;

Options options() {
  std::lock_guard<std::mutex> lk(g_opt_mu);
  return g_opt;
}

// ------------------------------------------------------------ device info

struct DeviceInfo {
  bool ok = false;
  int cus = 0;
  int occ[mk::kShapes][2][2] = {};  // fused occupancy per [shape][pt][ct] (workgroups per CU),
                                    // both variants
  int ag_occ[3][2] = {};  // AllGather+GEMM kernel occupancy per [shape][ct]
};
std::mutex g_dev_mu;
std::map<int, DeviceInfo> g_dev;

mk_status_t device_info(int dev, DeviceInfo& out) {
  std::lock_guard<std::mutex> lk(g_dev_mu);
  auto it = g_dev.find(dev);
  if (it != g_dev.end()) {
    out = it->second;
    return MK_OK;
  }
  hipDeviceProp_t p;
  hipError_t e = hipGetDeviceProperties(&p, dev);
  if (e != hipSuccess) return fail(MK_ERR_NO_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
  if (strncmp(p.gcnArchName, "gfx950", 6) != 0)
    return fail(MK_ERR_NO_DEVICE, "device %d is %s; this library is built for gfx950", dev,
                p.gcnArchName);
  DeviceInfo d;
  d.cus = p.multiProcessorCount;
  for (int s = 1; s < mk::kShapes; ++s)
    for (int pt = 0; pt < 2; ++pt)
      for (int ct = 0; ct < 2; ++ct) {
        // the persistent grid is sized from this count, so it holds for both
        // variants of the kernel (the lower of the two: the dynamic hand-over
        // kernel, or the 128x128 wave-specialised kernel's four streaming waves;
        // 64-wide tiles and 64x256 wave-specialised tiles have one)
        int n = 1 << 30;
        const int variants =
            s == mk::SHAPE_256 || s == mk::SHAPE_128 || s == mk::SHAPE_WS128 ? 2 : 1;
        for (int v = 0; v < variants; ++v) {
          int m = 0;
          e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
              &m, mk::fused_kernel_ptr(s, pt, ct, v), mk::shape_threads(s, v), 0);
          if (e != hipSuccess || m < 1)
            return fail(MK_ERR_HIP, "occupancy query failed: %s", hipGetErrorString(e));
          n = m < n ? m : n;
        }
        d.occ[s][pt][ct] = n;
      }
  for (int s = 1; s <= 2; ++s)
    for (int ct = 0; ct < 2; ++ct) {
      int n = 0;
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, mk::ag_kernel_ptr(s, ct),
                                                       mk::kThreadsHost, 0);
      if (e != hipSuccess || n < 1)
        return fail(MK_ERR_HIP, "occupancy query failed: %s", hipGetErrorString(e));
      d.ag_occ[s][ct] = n;
    }
  d.ok = true;
  g_dev[dev] = d;
  out = d;
  return MK_OK;
}

// ------------------------------------------------------------ workspaces

struct Workspace {
  int device = 0;
  float* P = nullptr;
  size_t P_elems = 0;
  int* flags = nullptr;
  int flags_cap = 0;
  int* ag_landed = nullptr;  // AllGather+GEMM piece flags (zero between calls)
  int ag_cap = 0;
  unsigned long long* slots = nullptr;
  int epoch = 0;
  unsigned long long handoffs = 0;  // calls of the flag hand-off microbenchmark
  // two-stream schedule: the reduce stream and its events (created on first use)
  hipStream_t s2 = nullptr;
  hipEvent_t ev[MK_MAX_CHUNKS + 1] = {};
  // ... and, with MK_OPT_STREAM_CU_SPLIT, the CU-masked GEMM and reduce streams
  // for the split they were made for, and the event that orders the GEMM
  // stream after the caller's stream
  hipStream_t sg_mask = nullptr, sr_mask = nullptr;
  int64_t mask_split = 0;
  hipEvent_t ev_start = nullptr;
};
std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, Workspace*> g_ws;

void free_ws(Workspace* w) {
  for (hipEvent_t e : w->ev)
    if (e) (void)hipEventDestroy(e);
  if (w->s2) (void)hipStreamDestroy(w->s2);
  if (w->sg_mask) (void)hipStreamDestroy(w->sg_mask);
  if (w->sr_mask) (void)hipStreamDestroy(w->sr_mask);
  if (w->ev_start) (void)hipEventDestroy(w->ev_start);
  if (w->P) (void)hipFree(w->P);
  if (w->flags) (void)hipFree(w->flags);
  if (w->ag_landed) (void)hipFree(w->ag_landed);
  if (w->slots) (void)hipFree(w->slots);
  delete w;
}

// Every workspace (and the streams and events it owns, CU-masked ones
// included) is released when the process exits normally, before the HIP
// runtime's own teardown: the handler is registered after the runtime has
// initialised, and exit handlers run in reverse order of registration.
void release_all_workspaces() {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  for (auto& kv : g_ws) {
    (void)hipSetDevice(kv.first.first);
    free_ws(kv.second);
  }
  g_ws.clear();
}
std::once_flag g_exit_once;

// Returns the workspace of (dev, stream) with room for P_elems partials and
// n_tiles flags; caller holds g_ws_mu.
mk_status_t get_ws(int dev, hipStream_t s, size_t P_elems, int n_tiles, Workspace** out) {
  auto key = std::make_pair(dev, s);
  Workspace* w;
  auto it = g_ws.find(key);
  if (it == g_ws.end()) {
    std::call_once(g_exit_once, [] { std::atexit(release_all_workspaces); });
    w = new Workspace();
    w->device = dev;
    hipError_t e = hipMalloc(&w->slots, sizeof(unsigned long long) * mk::S_COUNT * mk::kSlotWords);
    if (e != hipSuccess) {
      delete w;
      return fail(MK_ERR_WORKSPACE, "workspace control words: %s", hipGetErrorString(e));
    }
    e = mk::launch_ws_init(nullptr, 0, w->slots, s);
    if (e != hipSuccess) {
      free_ws(w);
      return hip_fail(e, "workspace init");
    }
    g_ws[key] = w;
  } else {
    w = it->second;
  }
  if (n_tiles > w->flags_cap || P_elems > w->P_elems) {
    // Growing: earlier calls on this stream may still use the old buffers.
    hipError_t e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  }
  if (n_tiles > w->flags_cap) {
    if (w->flags) (void)hipFree(w->flags);
    w->flags = nullptr;
    w->flags_cap = 0;
    int cap = n_tiles < 1024 ? 1024 : n_tiles;
    hipError_t e = hipMalloc(&w->flags, sizeof(int) * (size_t)cap);
    if (e != hipSuccess) return fail(MK_ERR_WORKSPACE, "tile flags: %s", hipGetErrorString(e));
    e = mk::launch_ws_init(w->flags, cap, nullptr, s);
    if (e != hipSuccess) return hip_fail(e, "flag init");
    w->flags_cap = cap;
  }
  if (P_elems > w->P_elems) {
    if (w->P) (void)hipFree(w->P);
    w->P = nullptr;
    w->P_elems = 0;
    hipError_t e = hipMalloc(&w->P, sizeof(float) * P_elems);
    if (e != hipSuccess)
      return fail(MK_ERR_WORKSPACE, "partial buffer of %zu floats: %s", P_elems, hipGetErrorString(e));
    w->P_elems = P_elems;
  }
  *out = w;
  return MK_OK;
}

// ------------------------------------------------------------ validation

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

size_t dt_size(int dt) { return dt == MK_DT_F32 ? 4 : 2; }

// Checks everything that can be checked without the GPU.
mk_status_t validate(const void* A, const void* B, const void* peers, int n_peers, void* C,
                     int64_t M, int64_t N, int64_t K, int peer_dtype, int c_dtype) {
  if (M < 0 || N < 0 || K < 0) return fail(MK_ERR_INVALID_ARG, "negative size M=%lld N=%lld K=%lld",
                                           (long long)M, (long long)N, (long long)K);
  if (n_peers < 0 || n_peers > MK_MAX_PEERS)
    return fail(MK_ERR_INVALID_ARG, "n_peers=%d outside [0, %d]", n_peers, MK_MAX_PEERS);
  if (peer_dtype != MK_DT_BF16 && peer_dtype != MK_DT_F32)
    return fail(MK_ERR_INVALID_ARG, "peer_dtype=%d", peer_dtype);
  if (c_dtype != MK_DT_BF16 && c_dtype != MK_DT_F32)
    return fail(MK_ERR_INVALID_ARG, "c_dtype=%d", c_dtype);
  if (N % 8 != 0 || K % 8 != 0)
    return fail(MK_ERR_UNSUPPORTED, "N=%lld and K=%lld must be multiples of 8", (long long)N,
                (long long)K);
  // The reducers address a tile's rows (at most 256) with 32-bit byte offsets
  // from the tile's first element: 256 rows of N fp32 values must stay below 4 GiB.
  if (N > ((int64_t)1 << 22))
    return fail(MK_ERR_UNSUPPORTED, "N=%lld exceeds 4194304", (long long)N);
  const int64_t lim = (int64_t)1 << 40;
  if (M > lim || N > lim || K > lim || (M > 0 && N > lim / M) || (M > 0 && K > lim / M) ||
      (N > 0 && K > lim / N) || (n_peers > 0 && M * N > lim / n_peers))
    return fail(MK_ERR_UNSUPPORTED, "sizes too large");
  const size_t a_bytes = (size_t)(M * K) * 2, b_bytes = (size_t)(K * N) * 2;
  const size_t p_bytes = (size_t)n_peers * (size_t)(M * N) * dt_size(peer_dtype);
  const size_t c_bytes = (size_t)(M * N) * dt_size(c_dtype);
  if (a_bytes && !A) return fail(MK_ERR_INVALID_ARG, "A is NULL");
  if (b_bytes && !B) return fail(MK_ERR_INVALID_ARG, "B is NULL");
  if (p_bytes && !peers) return fail(MK_ERR_INVALID_ARG, "peers is NULL with n_peers=%d", n_peers);
  if (c_bytes && !C) return fail(MK_ERR_INVALID_ARG, "C is NULL");
  const void* ptrs[] = {A, B, peers, C};
  const char* names[] = {"A", "B", "peers", "C"};
  for (int i = 0; i < 4; ++i)
    if (((uintptr_t)ptrs[i]) % 16 != 0) return fail(MK_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
  if (overlaps(C, c_bytes, A, a_bytes) || overlaps(C, c_bytes, B, b_bytes) ||
      overlaps(C, c_bytes, peers, p_bytes))
    return fail(MK_ERR_INVALID_ARG, "C overlaps an input");
  return MK_OK;
}

// The same checks for a GEMM+ReduceScatter share: A [M,K], B [K,N], peers
// [n_peers, own, N], C [own, N] (own = own_m1 - own_m0 rows), send [M, N] of the
// peer type (not read or written when every row is owned).
mk_status_t validate_rs(const void* A, const void* B, const void* peers, int n_peers, void* C,
                        void* send, int64_t M, int64_t N, int64_t K, int64_t own_m0,
                        int64_t own_m1, int peer_dtype, int c_dtype) {
  if (own_m0 < 0 || own_m1 < own_m0 || own_m1 > M)
    return fail(MK_ERR_INVALID_ARG, "owned rows [%lld, %lld) outside [0, %lld]", (long long)own_m0,
                (long long)own_m1, (long long)M);
  const int64_t own = own_m1 - own_m0;
  // A, B, peers and C as for an AllReduce share of `own` rows; then A's other rows
  mk_status_t st = validate(A, B, peers, n_peers, C, own, N, K, peer_dtype, c_dtype);
  if (st != MK_OK) return st;
  if (own < M) {  // send [M, N] in the peer type, like a C of all M rows
    st = validate(A, B, nullptr, 0, send, M, N, K, peer_dtype, peer_dtype);
    if (st != MK_OK) return st;
  }
  const size_t a_bytes = (size_t)(M * K) * 2;
  const size_t p_bytes = (size_t)n_peers * (size_t)(own * N) * dt_size(peer_dtype);
  const size_t c_bytes = (size_t)(own * N) * dt_size(c_dtype);
  const size_t s_bytes = own < M ? (size_t)(M * N) * dt_size(peer_dtype) : 0;
  if (s_bytes && !send) return fail(MK_ERR_INVALID_ARG, "send is NULL");
  if (overlaps(C, c_bytes, A, a_bytes) || overlaps(send, s_bytes, peers, p_bytes) ||
      overlaps(send, s_bytes, C, c_bytes))
    return fail(MK_ERR_INVALID_ARG, "C or send overlaps another argument");
  return MK_OK;
}

// The wave-specialised kernel's automatic choice: for shapes whose peer stream
// (at HBM peak) takes at least 1.8 times their GEMM (at matrix-core peak), with
// a 64x256 tile for every compute unit; 64x256 tiles (512-byte pieces of peer
// rows) from four times on, 128x128 tiles (fewer A and B bytes per output)
// below. Returns the shape, or 0 for the other schedules. Where the GEMM weighs
// more, the overlap gains less than the smaller tiles cost. Measured on MI355X,
// us per call (stream/GEMM ratio; 256x256 tiles in place / 64x256 / 128x128
// with 64-deep k-tiles in three stages and, with 15 peers, four streaming
// waves; same machine):
//   16384x8192x512 P=16 (9.8)   928 / 802 / 902     8192x8192x512 P=16 (9.8)  501 / 412 / 446
//   16384x8192x1024 P=16 (4.9) 1010 / 923 / 989     4096x8192x1024 P=16 (4.9) 273 / 245 / 234
//   4096x8192x1792 P=16 (2.8)   311 / 313 / 273     8192x8192x1024 P=8 (2.4)  336 / 328 / 291
//   8192x16384x1024 P=8 (2.4)   608 / 648 / 571     4096x8192x2560 P=16 (1.95) 356 / 387 / 334
//   4096x8192x3584 P=16 (1.4)   399 / 483 / 403     8192x8192x2048 P=8 (1.2)  435 / 516 / 442
int ws_pays(int64_t M, int64_t N, int64_t K, int n_peers, int peer_dtype, int c_dtype, int cus) {
  const double t_stream =
      (double)M * (double)N * (n_peers * (double)dt_size(peer_dtype) + dt_size(c_dtype)) / 8.0e12;
  const double t_gemm = 2.0 * (double)M * (double)N * (double)K / 2.5e15;
  const int64_t tiles = ((M + 63) / 64) * ((N + 255) / 256);
  if (tiles < cus || t_stream < 1.8 * t_gemm) return 0;
  return t_stream >= 4.0 * t_gemm ? mk::SHAPE_WS : mk::SHAPE_WS128;
}

// 256x256 tiles (one workgroup per CU) whenever they still give every CU a tile:
// they need half the L2 traffic per flop of 128x128 tiles. Otherwise 128x128
// tiles (two workgroups per CU) while those still give every CU a tile. Measured
// on the 16384x8192x512 shape with 15 peers (interleaved runs on one box):
// 256-tiles 969-979 us, 128-tiles 1073-1081 us. Shapes with fewer 128-tiles than
// CUs take 64x64 tiles, each reduced in place by the one workgroup that computes
// it (allow64: the AllReduce paths; ReduceScatter keeps 128 and up). Measured on
// the 128x8192x1792 shard with 15 peers: 19.5 us against 33.6 us for 128-tiles
// with early reduce and k-halves (baselines 22.7 and 34.6 us); 256x512x512 with 3
// fp32 peers: 9.2 against 19.4 us (baselines 11.6 and 13.6 us).
//
// ws: the call may run the wave-specialised kernel (SHAPE_WS: the fused
// AllReduce without telemetry, K > 0, a peer count whose tiles can be reduced in
// place at two waves per SIMD); auto_ws: the automatic choice may take it (no
// explicit reducer count, in-place policy or early reduce).
int pick_shape(int64_t M, int64_t N, int64_t K, int n_peers, int peer_dtype, int c_dtype, int cus,
               bool allow64, bool ws, bool auto_ws) {
  (void)c_dtype;
  ws = ws && allow64 && K > 0 && mk::inplace_supported(2, (int)dt_size(peer_dtype), n_peers);
  int64_t forced = options().tile_shape;
  if (forced == mk::SHAPE_256 || forced == mk::SHAPE_128) return (int)forced;
  if (forced == mk::SHAPE_64) return allow64 ? mk::SHAPE_64 : mk::SHAPE_128;
  if ((forced == mk::SHAPE_WS || forced == mk::SHAPE_WS128) && ws) return (int)forced;
  const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
  const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
  if (forced == mk::SHAPE_AUTO && ws && auto_ws)
    if (int s = ws_pays(M, N, K, n_peers, peer_dtype, c_dtype, cus)) return s;
  if (t256 >= cus) return mk::SHAPE_256;
  return t128 >= cus || !allow64 ? mk::SHAPE_128 : mk::SHAPE_64;
}

// Host roofline seed for the controller: the reducers' share of the work when
// the reduce streams at HBM speed and the GEMM runs at matrix-core peak.
float seed_share(int64_t M, int64_t N, int64_t K, int n_peers, int peer_dtype, int c_dtype) {
  double flops = 2.0 * (double)M * (double)N * (double)K;
  double red_bytes = (double)M * (double)N * (4.0 + n_peers * (double)dt_size(peer_dtype) + dt_size(c_dtype));
  double t_mfma = flops / 2.5e15, t_hbm = red_bytes / 8.0e12;
  if (t_mfma + t_hbm <= 0) return 0.5f;
  return (float)(t_hbm / (t_hbm + t_mfma));
}

struct Launch {
  int dev;
  DeviceInfo info;
  int shape;
  int64_t tiles_m, tiles_n;
  int64_t K;
};

// Whether reducers sum a unit's peers before its tile is finished (early
// reduce), from MK_OPT_EARLY: automatic (-1) turns it on for shapes whose tiles
// and reduce units all fit in one round of resident workgroups (one per tile
// and one per unit), e.g. a decode-sized shard; with more tiles than that,
// reducers would sum one unit's peers and then wait for a tile that is still
// far from done. Only peer counts with a compile-time ring.
bool early_reduce(const Launch& L, int n_peers, int peer_dtype, int c_dtype) {
  const int64_t opt = options().early;
  const int occ = L.shape == mk::SHAPE_256 ? 1 : 2;
  // 64-wide tiles are always reduced in place
  if (opt == 0 || n_peers < 1 || L.shape == mk::SHAPE_64 || mk::is_ws(L.shape) ||
      !mk::inplace_supported(occ, (int)dt_size(peer_dtype), n_peers))
    return false;
  if (opt > 0) return true;
  const int64_t T = L.tiles_m * L.tiles_n;
  const int64_t full = (int64_t)L.info.cus * L.info.occ[L.shape][peer_dtype][c_dtype];
  return T * (1 + mk::shape_bm(L.shape) / 64) <= full;
}

// K-split of an early-reduce call (MK_OPT_KSPLIT): automatic (-1) computes each
// tile as two k-halves when the call has early reduce, K is a multiple of 64 and
// at least 512, and every item (two per tile) and reduce unit still fits one
// round of resident workgroups. A decode-sized tile is otherwise one workgroup
// streaming the tile's whole B panel at one compute unit's rate. Measured on the
// 128x8192x1792 shard with 15 peers: unsplit 38.0-40.4 us, two parts 32.2-33.7 us,
// four parts 36.4 us (two-kernel baseline 34.5-34.9 us); 256x512x512 with 3 fp32
// peers: 19.3-19.6 -> 18.2-18.3 us.
int ksplit_of(const Launch& L, int n_peers, int peer_dtype, int c_dtype) {
  const int64_t opt = options().ksplit;
  if (opt == 1 || !early_reduce(L, n_peers, peer_dtype, c_dtype) || L.K % 64 != 0) return 1;
  if (opt == 2) return 2;
  const int64_t T = L.tiles_m * L.tiles_n;
  const int64_t full = (int64_t)L.info.cus * L.info.occ[L.shape][peer_dtype][c_dtype];
  return L.K >= 512 && T * (2 + mk::shape_bm(L.shape) / 64) <= full ? 2 : 1;
}

// Persistent grid of the fused kernel: every resident workgroup slot (compute
// units times workgroups per unit), but no more than two workgroups per tile
// (with early reduce: one per tile, or two with a k-split, plus one per reduce
// unit), rounded up to a
// multiple of the XCD count, so that a call with few tiles does not start
// hundreds of workgroups that only find no work and leave.
int fused_grid_size(const Launch& L, int n_peers, int peer_dtype, int c_dtype) {
  const int full = L.info.cus * L.info.occ[L.shape][peer_dtype][c_dtype];
  int n_xcd = L.info.cus / 32;
  if (n_xcd < 1) n_xcd = 1;
  const int64_t T = L.tiles_m * L.tiles_n;
  // 64-wide tiles are all reduced in place: one workgroup per tile (at least one
  // per XCD, as for every shape)
  if (L.shape == mk::SHAPE_64) {
    const int64_t g = T < n_xcd ? n_xcd : T;
    return g < full ? (int)g : full;
  }
  // wave-specialised: one workgroup per compute unit, at most one per tile
  if (mk::is_ws(L.shape)) return T < full ? (int)(T > 0 ? T : 1) : full;
  int64_t want = early_reduce(L, n_peers, peer_dtype, c_dtype)
                     ? T * (ksplit_of(L, n_peers, peer_dtype, c_dtype) + mk::shape_bm(L.shape) / 64)
                     : 2 * T;
  want = (want + n_xcd - 1) / n_xcd * n_xcd;
  if (want < n_xcd) want = n_xcd;
  return want < full ? (int)want : full;
}

// Grid of the AllGather landing copy for `elems` elements: two 8-element
// chunks per thread, at most 8 workgroups per compute unit (grid-stride beyond).
int copy_grid(int64_t elems, int cus) {
  const int64_t chunks = elems / 8;
  int64_t grid = (chunks + 2 * 256 - 1) / (2 * 256);
  const int64_t cap = (int64_t)cus * 8;
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  return (int)grid;
}

// Grid of the reduce kernel for `elems` output elements: one workgroup per
// compute unit, fewer when there are fewer than 256 chunks of 8 elements per
// workgroup. Each thread keeps its next chunk's loads in flight while it sums
// one; on MI355X one such workgroup per compute unit streamed the attention
// shape's 15 peers at 6.2 TB/s, against 5.6-5.8 TB/s with 4 or 8 per unit.
int reduce_grid(int64_t elems, int cus) {
  const int64_t chunks = elems / 8;
  int64_t grid = (chunks + 256 - 1) / 256;
  if (grid > cus) grid = cus;
  if (grid < 1) grid = 1;
  return (int)grid;
}

// Grid of a ReduceScatter share: as for the AllReduce share without early
// reduce (at most two workgroups per tile).
int rs_grid_size(const Launch& L, int peer_dtype, int c_dtype) {
  const int full = L.info.cus * L.info.occ[L.shape][peer_dtype][c_dtype];
  int n_xcd = L.info.cus / 32;
  if (n_xcd < 1) n_xcd = 1;
  int64_t want = 2 * L.tiles_m * L.tiles_n;
  want = (want + n_xcd - 1) / n_xcd * n_xcd;
  if (want < n_xcd) want = n_xcd;
  return want < full ? (int)want : full;
}

mk_status_t prepare(int64_t M, int64_t N, int64_t K, int n_peers, int peer_dtype, int c_dtype,
                    Launch& L, bool allow64 = true, bool ws = false, bool auto_ws = false) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MK_ERR_NO_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  mk_status_t st = device_info(dev, L.info);
  if (st != MK_OK) return st;
  L.dev = dev;
  L.K = K;
  L.shape = pick_shape(M, N, K, n_peers, peer_dtype, c_dtype, L.info.cus, allow64, ws, auto_ws);
  L.tiles_m = (M + mk::shape_bm(L.shape) - 1) / mk::shape_bm(L.shape);
  L.tiles_n = (N + mk::shape_bn(L.shape) - 1) / mk::shape_bn(L.shape);
  if (L.tiles_m * L.tiles_n > (1 << 30)) return fail(MK_ERR_UNSUPPORTED, "too many tiles");
  return MK_OK;
}


// ------------------------------------------------------------ AllGather+GEMM share

// A_local [Ms,K], peers_A [n_peers,Ms,K], A_full [P*Ms,K], B [K,N], C [P*Ms,N].
mk_status_t validate_ag(const void* A_local, const void* peers_A, int n_peers, void* A_full,
                        const void* B, void* C, int64_t Ms, int64_t N, int64_t K, int rank,
                        int c_dtype) {
  if (Ms < 0 || N < 0 || K < 0)
    return fail(MK_ERR_INVALID_ARG, "negative size Ms=%lld N=%lld K=%lld", (long long)Ms,
                (long long)N, (long long)K);
  if (n_peers < 0 || n_peers > MK_MAX_PEERS)
    return fail(MK_ERR_INVALID_ARG, "n_peers=%d outside [0, %d]", n_peers, MK_MAX_PEERS);
  if (rank < 0 || rank > n_peers)
    return fail(MK_ERR_INVALID_ARG, "rank=%d outside [0, %d]", rank, n_peers);
  if (c_dtype != MK_DT_BF16 && c_dtype != MK_DT_F32)
    return fail(MK_ERR_INVALID_ARG, "c_dtype=%d", c_dtype);
  if (N % 8 != 0 || K % 8 != 0)
    return fail(MK_ERR_UNSUPPORTED, "N=%lld and K=%lld must be multiples of 8", (long long)N,
                (long long)K);
  if (Ms % 128 != 0)
    return fail(MK_ERR_UNSUPPORTED, "Ms=%lld must be a multiple of 128", (long long)Ms);
  if (N > ((int64_t)1 << 22))
    return fail(MK_ERR_UNSUPPORTED, "N=%lld exceeds 4194304", (long long)N);
  const int64_t M = (int64_t)(n_peers + 1) * Ms;
  const int64_t lim = (int64_t)1 << 40;
  if (M > lim || K > lim || (M > 0 && N > lim / M) || (M > 0 && K > lim / M) ||
      (N > 0 && K > lim / N))
    return fail(MK_ERR_UNSUPPORTED, "sizes too large");
  const size_t l_bytes = (size_t)(Ms * K) * 2, p_bytes = (size_t)n_peers * l_bytes;
  const size_t f_bytes = (size_t)(M * K) * 2, b_bytes = (size_t)(K * N) * 2;
  const size_t c_bytes = (size_t)(M * N) * dt_size(c_dtype);
  if (l_bytes && !A_local) return fail(MK_ERR_INVALID_ARG, "A_local is NULL");
  if (p_bytes && !peers_A) return fail(MK_ERR_INVALID_ARG, "peers_A is NULL with n_peers=%d", n_peers);
  if (f_bytes && !A_full) return fail(MK_ERR_INVALID_ARG, "A_full is NULL");
  if (b_bytes && !B) return fail(MK_ERR_INVALID_ARG, "B is NULL");
  if (c_bytes && !C) return fail(MK_ERR_INVALID_ARG, "C is NULL");
  const void* ptrs[] = {A_local, peers_A, A_full, B, C};
  const char* names[] = {"A_local", "peers_A", "A_full", "B", "C"};
  for (int i = 0; i < 5; ++i)
    if (((uintptr_t)ptrs[i]) % 16 != 0) return fail(MK_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
  if (overlaps(A_full, f_bytes, A_local, l_bytes) || overlaps(A_full, f_bytes, peers_A, p_bytes) ||
      overlaps(A_full, f_bytes, B, b_bytes) || overlaps(A_full, f_bytes, C, c_bytes))
    return fail(MK_ERR_INVALID_ARG, "A_full overlaps another argument");
  if (overlaps(C, c_bytes, A_local, l_bytes) || overlaps(C, c_bytes, peers_A, p_bytes) ||
      overlaps(C, c_bytes, B, b_bytes))
    return fail(MK_ERR_INVALID_ARG, "C overlaps an input");
  return MK_OK;
}

// Tile shape of an AllGather+GEMM share: bands never straddle two shards, so
// 256-row tiles need Ms a multiple of 256; they are taken when at least half of
// the CUs get a tile (on the 4096x3584x8192 shape, 224 tiles of 256x256 ran in
// 246-253 us, 896 tiles of 128x128 in 294-342 us).
int ag_shape(int64_t Ms, int P, int64_t N, int cus) {
  const int64_t forced = options().tile_shape;
  const bool ok256 = Ms % 256 == 0;
  if (forced == mk::SHAPE_128 || (forced == mk::SHAPE_256 && !ok256)) return mk::SHAPE_128;
  if (forced == mk::SHAPE_256) return mk::SHAPE_256;
  const int64_t t256 = (int64_t)P * (Ms / 256) * ((N + 255) / 256);
  return ok256 && 2 * t256 >= cus ? mk::SHAPE_256 : mk::SHAPE_128;
}

// Persistent grid of the AllGather+GEMM kernel: one workgroup per tile plus
// four landing workgroups per XCD, at most every resident slot, a multiple of
// the XCD count.
int ag_grid_size(const DeviceInfo& info, int shape, int c_dtype, int64_t T) {
  const int full = info.cus * info.ag_occ[shape][c_dtype];
  int n_xcd = info.cus / 32;
  n_xcd = n_xcd < 1 ? 1 : (n_xcd > mk::kMaxXcd ? mk::kMaxXcd : n_xcd);
  const int64_t want = (T + 4 * n_xcd + n_xcd - 1) / n_xcd * n_xcd;
  return want < full ? (int)want : full / n_xcd * n_xcd;
}


// ------------------------------------------------------------ fused AllReduce plan

// Arguments of one fused AllReduce call, checked.
struct ArCall {
  const void *A, *B, *peers;
  void* C;
  int64_t M, N, K;
  int n_peers, peer_dtype, c_dtype, n_reduce_wg;
  void* telemetry;
  Launch L;
};

// The automatic choice of the wave-specialised kernel leaves a call alone that
// names its schedule: a reducer count, an in-place policy, early reduce or a k-split.
bool ws_auto_allowed(int n_reduce_wg) {
  const Options o = options();
  return n_reduce_wg == MK_ADAPTIVE && o.inplace == -1 && o.early == -1 && o.ksplit == -1;
}

mk_status_t ar_prepare(const void* A, const void* B, const void* peers, int n_peers, void* C,
                       int64_t M, int64_t N, int64_t K, int peer_dtype, int c_dtype,
                       int n_reduce_wg, void* telemetry, ArCall& c) {
  mk_status_t st = validate(A, B, peers, n_peers, C, M, N, K, peer_dtype, c_dtype);
  if (st != MK_OK) return st;
  if (n_reduce_wg < MK_ADAPTIVE) return fail(MK_ERR_INVALID_ARG, "n_reduce_wg=%d", n_reduce_wg);
  if (((uintptr_t)telemetry) % 16 != 0) return fail(MK_ERR_INVALID_ARG, "telemetry not 16-byte aligned");
  st = prepare(M, N, K, n_peers, peer_dtype, c_dtype, c.L, true, telemetry == nullptr,
               ws_auto_allowed(n_reduce_wg));
  if (st != MK_OK) return st;
  c.A = A;
  c.B = B;
  c.peers = peers;
  c.C = C;
  c.M = M;
  c.N = N;
  c.K = K;
  c.n_peers = n_peers;
  c.peer_dtype = peer_dtype;
  c.c_dtype = c_dtype;
  c.n_reduce_wg = n_reduce_wg;
  c.telemetry = telemetry;
  // the reducer count is checked against the grid of the default plan (the
  // wave-specialised kernel has no reducer workgroups and ignores it)
  const int G = fused_grid_size(c.L, n_peers, peer_dtype, c_dtype);
  if (!mk::is_ws(c.L.shape) && n_reduce_wg > G - 1)
    return fail(MK_ERR_INVALID_ARG, "n_reduce_wg=%d outside [0, %d]", n_reduce_wg, G - 1);
  return MK_OK;
}

// Whether every tile of every XCD queue is reduced in place.
bool T_inplace_all(const mk::FusedArgs& a, bool inpl_ok) {
  if (!inpl_ok) return false;
  for (int xi = 0; xi < a.n_xcd; ++xi) {
    const int cnt = mk::xcd_tiles(a.T, a.n_xcd, xi);
    if (mk::xcd_inplace(cnt, a.n_inplace, inpl_ok) != cnt) return false;
  }
  return true;
}

// Decides the grid, the in-place policy, early reduce, the k-split and the
// controller's seed and cap of a call, and fills every argument of the fused
// kernel but the workspace (P, flags, slots, epoch). all_inplace: every tile
// reduced in place by the workgroup that computed it (no partial in memory, no
// early reduce or k-split), for peer counts that allow it.
mk_status_t ar_plan(const ArCall& c, bool all_inplace, mk::FusedArgs& a) {
  const Launch& L = c.L;
  const int64_t M = c.M, N = c.N, K = c.K;
  const int n_peers = c.n_peers, peer_dtype = c.peer_dtype, c_dtype = c.c_dtype;
  const Options opt = options();
  const bool inpl_ok =
      mk::inplace_supported(L.shape == mk::SHAPE_256 ? 1 : 2, dt_size(peer_dtype), n_peers);
  if (all_inplace && !inpl_ok)
    return fail(MK_ERR_UNSUPPORTED, "tiles of %d peers of this type cannot be reduced in place",
                n_peers);
  const bool early = !all_inplace && early_reduce(L, n_peers, peer_dtype, c_dtype);
  const int ks = all_inplace ? 1 : ksplit_of(L, n_peers, peer_dtype, c_dtype);
  int G;
  {
    const int full = L.info.cus * L.info.occ[L.shape][peer_dtype][c_dtype];
    int n_xcd = L.info.cus / 32;
    if (n_xcd < 1) n_xcd = 1;
    const int64_t T = L.tiles_m * L.tiles_n;
    int64_t want = early ? T * (ks + mk::shape_bm(L.shape) / 64) : 2 * T;
    want = (want + n_xcd - 1) / n_xcd * n_xcd;
    if (want < n_xcd) want = n_xcd;
    G = want < full ? (int)want : full;
    // 64-wide tiles are all reduced in place: one workgroup per tile (at least one
    // per XCD, as for every shape)
    if (L.shape == mk::SHAPE_64) {
      const int64_t g = T < n_xcd ? n_xcd : T;
      G = g < full ? (int)g : full;
    }
    if (mk::is_ws(L.shape)) G = T < full ? (int)(T > 0 ? T : 1) : full;
  }
  if (!mk::is_ws(L.shape) && c.n_reduce_wg > G - 1)
    return fail(MK_ERR_INVALID_ARG, "n_reduce_wg=%d outside [0, %d]", c.n_reduce_wg, G - 1);
  const int T = (int)(L.tiles_m * L.tiles_n);
  memset(&a, 0, sizeof a);
  a.A = (const uint16_t*)c.A;
  a.B = (const uint16_t*)c.B;
  a.peers = c.peers;
  a.C = c.C;
  a.tel = (mk_telemetry_t*)c.telemetry;
  a.M = M;
  a.N = N;
  a.K = K;
  a.n_peers = n_peers;
  a.tiles_m = (int)L.tiles_m;
  a.tiles_n = (int)L.tiles_n;
  a.T = T;
  a.G = G;
  a.seed_x = seed_share(M, N, K, n_peers, peer_dtype, c_dtype);
  if (c.n_reduce_wg == MK_ADAPTIVE) {
    a.adaptive = 1;
    int t0 = (int)lrintf(a.seed_x * (float)G);
    a.init_target = t0 < 1 ? 1 : (t0 > G - 1 ? G - 1 : t0);
  } else {
    a.adaptive = 0;
    a.init_target = c.n_reduce_wg;
  }
  a.ctrl_period = opt.ctrl_period < 1 ? 1 : (int)opt.ctrl_period;
  a.withhold_tile = (int)opt.withhold_tile;
  a.spin_limit = (unsigned long long)(opt.spin_timeout_us < 1 ? 1 : opt.spin_timeout_us) * 100ull;
  // tiles are queued per XCD where the device's layout allows it (queue_plan)
  mk::queue_plan(L.info.cus, G, (int)opt.flag_scope, a.n_xcd, a.flag_scope);
  a.shared_lines = N % 32 != 0 ? 1 : 0;  // partial rows not whole 128-byte lines
  a.reducer_cap = (int)opt.reducer_cap;
  if (a.reducer_cap <= 0) {
    // Compute units that saturate HBM with the reduce stream: about 5.5 TB/s
    // sustained over about 40 GB/s, the most one compute unit streams (measured
    // on MI355X whatever the loads in flight), times the workgroups per compute
    // unit; a multiple of the XCD count.
    const int occ = L.shape == mk::SHAPE_256 ? 1 : 2;  // workgroups per compute unit
    int cap = (int)ceil(5.5e12 / 40e9) * occ;
    cap = (cap + a.n_xcd - 1) / a.n_xcd * a.n_xcd;
    a.reducer_cap = cap < G - 1 ? cap : G - 1;
  }
  if (a.adaptive && a.init_target > a.reducer_cap) a.init_target = a.reducer_cap < 1 ? 1 : a.reducer_cap;
  // In-place tiles per XCD, counted from the end of the XCD's queue. Automatic
  // (-1): every tile, unless the call has early reduce (then every tile is handed
  // over). Measured on one MI355X (bench.py --sweep, 256 workgroups), a tile
  // handed to another workgroup only adds its partial's round trip through
  // memory: every tile in place took 315 us on 4096x8192x1792 with 15 peers
  // (against 320-326 us handing over the first quarter of each queue's first
  // round), 972 us on 16384x8192x512 and 1107 us on 8192^3 with 7 peers.
  // MK_OPT_INPLACE = -2 decides per tile instead (dynamic hand-over, below).
  a.early = early ? 1 : 0;
  if (all_inplace || mk::is_ws(L.shape)) {
    a.n_inplace = 1 << 30;
  } else if (opt.inplace < 0 && a.early) {
    a.n_inplace = 0;  // early reduce applies to tiles handed to reducers
  } else if (opt.inplace < 0) {
    a.n_inplace = 1 << 30;
  } else {
    a.n_inplace = (int)opt.inplace;
  }
  // Two k-halves only when every tile is handed to a reducer (an in-place tile
  // would reduce its own half-product).
  a.ksplit = a.early && a.n_inplace == 0 ? ks : 1;
  // Dynamic hand-over (MK_OPT_INPLACE = -2, without early reduce): every tile is
  // reduced in place or handed over when its GEMM ends, by the streaming slots
  // free then. The controller's target counts workgroups streaming a reduce, in
  // place or handed over, so all reduce work is its reducers' (T_r = T).
  a.dyn = opt.inplace == -2 && !all_inplace && !a.early && inpl_ok && L.shape != mk::SHAPE_64 &&
                  !mk::is_ws(L.shape)
              ? 1
              : 0;
  a.T_r = 0;
  if (a.dyn) {
    a.n_inplace = 0;
    a.T_r = T;
  } else {
    for (int xi = 0; xi < a.n_xcd; ++xi) {
      const int cnt = mk::xcd_tiles(a.T, a.n_xcd, xi);
      a.T_r += cnt - mk::xcd_inplace(cnt, a.n_inplace, inpl_ok);
    }
  }
  // With tiles reduced in place, compute workgroups do most of the reduce
  // themselves; a dedicated reducer takes a compute unit away from the GEMM and
  // competes with them for memory bandwidth (measured on the 4096x8192x1792
  // shape: 0 reducers 324 us, one per XCD 351 us, 64 348 us). The derived cap
  // is then zero: the adaptive controller keeps every workgroup computing while
  // GEMM tiles remain, and all of them drain the handed-over tiles.
  if (opt.reducer_cap <= 0 && a.T_r < a.T && !a.dyn) a.reducer_cap = 0;
  // With dynamic hand-over a tile beyond the streaming slots makes the partial's
  // round trip through memory; the target is left to the measured split of the
  // work rather than held under the HBM cap.
  if (opt.reducer_cap <= 0 && a.dyn) {
    a.reducer_cap = G - 1;
    if (a.adaptive) {
      int t0 = (int)lrintf(a.seed_x * (float)G);
      a.init_target = t0 < 1 ? 1 : (t0 > G - 1 ? G - 1 : t0);
    }
  }
  // One workgroup per tile with every tile in place: no claims or counters (no
  // telemetry either, which is what a telemetry buffer asks for).
  a.one_tile = !a.dyn && !a.early && T_inplace_all(a, inpl_ok) && T <= G && !c.telemetry &&
                       !mk::is_ws(L.shape)
                   ? 1
                   : 0;
  // Every tile in place with more tiles than one round of workgroups, 256x256
  // tiles: the in-place kernel, which deals the tiles in a fixed order and keeps
  // no claim or flag state (MK_OPT_STATIC_TILES).
  a.ws_wide = mk::ws_wide(L.shape, (int)dt_size(peer_dtype), n_peers) ? 1 : 0;
  a.static_tiles = !a.one_tile && !a.dyn && !a.early && a.ksplit == 1 &&
                           T_inplace_all(a, inpl_ok) && !c.telemetry &&
                           L.shape == mk::SHAPE_256 && opt.static_tiles >= 1
                       ? 1
                       : 0;
  // ... with eight waves where the tile-end rings fit two waves per SIMD
  a.waves8 = a.static_tiles && opt.static_tiles == 2 &&
                     mk::inplace_supported(2, (int)dt_size(peer_dtype), n_peers)
                 ? 1
                 : 0;
  // The seed share counts the in-place tiles' reduce as compute-side work.
  if (a.T > 0 && a.T_r < a.T) {
    double flops = 2.0 * (double)M * (double)N * (double)K;
    double red_bytes = (double)M * (double)N * (4.0 + n_peers * (double)dt_size(peer_dtype) + dt_size(c_dtype));
    double t_r = red_bytes * ((double)a.T_r / a.T) / 8.0e12;
    double t_c = flops / 2.5e15 + red_bytes * ((double)(a.T - a.T_r) / a.T) / 8.0e12;
    a.seed_x = (float)(t_r / (t_r + t_c));
    if (a.adaptive) {
      int it = (int)(a.seed_x * G + 0.5f);
      const int lo = a.reducer_cap < 1 ? a.reducer_cap : 1;
      it = it < lo ? lo : (it > a.reducer_cap ? a.reducer_cap : it);
      a.init_target = it;
    }
  }
  return MK_OK;
}

// 32-bit words of tile flags a call needs: its flags (tiles times k-parts), then,
// 8-byte aligned, one 64-bit publication slot per tile for dynamic hand-over.
int ar_flag_words(const mk::FusedArgs& a) {
  const int f = a.T * a.ksplit;
  return a.dyn ? (f + 1) / 2 * 2 + 2 * a.T : f;
}
unsigned long long* ar_pub_slots(const mk::FusedArgs& a, int* flags) {
  return a.dyn ? (unsigned long long*)(flags + (a.T * a.ksplit + 1) / 2 * 2) : nullptr;
}

// ------------------------------------------------------------ allocation-free workspace

// Per-device state of the fixed workspace: its device address (looked up once
// per device, with that device current), whether its flags and control words
// have been cleared, and the epoch of the last call.
struct Scratch {
  unsigned char* base = nullptr;
  bool ready = false;
  int epoch = 0;
};
std::mutex g_scratch_mu;
std::map<int, Scratch> g_scratch;

unsigned long long* scratch_slots(const Scratch& s) { return (unsigned long long*)s.base; }
int* scratch_flags(const Scratch& s) { return (int*)(s.base + mk::kScratchSlotBytes); }
float* scratch_partial(const Scratch& s) {
  return (float*)(s.base + mk::kScratchSlotBytes + mk::kScratchFlags * 4);
}

// Caller holds g_scratch_mu; `dev` is current.
mk_status_t scratch_of(int dev, Scratch** out) {
  Scratch& s = g_scratch[dev];
  if (!s.base) {
    void* p = nullptr;
    hipError_t e = mk::noalloc_scratch_address(&p);
    if (e != hipSuccess || !p) return hip_fail(e, "address of the allocation-free workspace");
    s.base = (unsigned char*)p;
  }
  *out = &s;
  return MK_OK;
}

}  // namespace

extern "C" {

mk_status_t mk_gemm_ar_local(const void* A, const void* B, const void* peers, int n_peers, void* C,
                             int64_t M, int64_t N, int64_t K, int peer_dtype, int c_dtype,
                             void* stream, int n_reduce_wg, void* telemetry) {
  ArCall c;
  mk_status_t st = ar_prepare(A, B, peers, n_peers, C, M, N, K, peer_dtype, c_dtype, n_reduce_wg,
                              telemetry, c);
  if (st != MK_OK || M == 0 || N == 0) return st;
  mk::FusedArgs a;
  st = ar_plan(c, false, a);
  if (st != MK_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  std::lock_guard<std::mutex> lk(g_ws_mu);
  Workspace* w = nullptr;
  // partial slices and flags per tile, and the publication slots (8 bytes per
  // tile, after the flags) of dynamic hand-over
  st = get_ws(c.L.dev, s, (size_t)(M * N) * a.ksplit, ar_flag_words(a), &w);
  if (st != MK_OK) return st;
  if (++w->epoch >= 0x7FFFFFFF) {  // flags hold old epochs: restart them from zero
    hipError_t e = mk::launch_ws_init(w->flags, w->flags_cap, nullptr, s);
    if (e != hipSuccess) return hip_fail(e, "flag reset");
    w->epoch = 1;
  }
  a.P = w->P;
  a.flags = w->flags;
  a.pub = ar_pub_slots(a, w->flags);
  a.slots = w->slots;
  a.epoch = w->epoch;
  hipError_t e = mk::launch_fused(c.L.shape, peer_dtype, c_dtype, a, s);
  if (e != hipSuccess) return hip_fail(e, "fused kernel launch");
  return MK_OK;
}

mk_status_t mk_gemm_ar_local_noalloc(const void* A, const void* B, const void* peers,
                                     int n_peers, void* C, int64_t M, int64_t N, int64_t K,
                                     int peer_dtype, int c_dtype, void* stream, int n_reduce_wg,
                                     void* telemetry) {
  ArCall c;
  mk_status_t st = ar_prepare(A, B, peers, n_peers, C, M, N, K, peer_dtype, c_dtype, n_reduce_wg,
                              telemetry, c);
  if (st != MK_OK || M == 0 || N == 0) return st;
  mk::FusedArgs a;
  st = ar_plan(c, false, a);
  if (st != MK_OK) return st;
  // The default plan needs the partial of every handed-over tile ([M, N] fp32 per
  // k-part); beyond the fixed partial region every tile is reduced in place.
  const size_t part_bytes = a.T_r > 0 ? (size_t)(M * N) * a.ksplit * 4 : 0;
  if (part_bytes > mk::kScratchPartialBytes) {
    st = ar_plan(c, true, a);
    if (st != MK_OK)
      return fail(MK_ERR_UNSUPPORTED,
                  "the partial of this call needs %zu bytes, more than the %zu of the "
                  "allocation-free workspace, and %s", part_bytes,
                  (size_t)mk::kScratchPartialBytes, mk_last_error());
  }
  if ((size_t)ar_flag_words(a) > mk::kScratchFlags)
    return fail(MK_ERR_UNSUPPORTED, "%d tiles x %d k-parts exceed the %zu tile flags of the "
                "allocation-free workspace", a.T, a.ksplit, (size_t)mk::kScratchFlags);
  hipStream_t s = (hipStream_t)stream;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  Scratch* sc = nullptr;
  st = scratch_of(c.L.dev, &sc);
  if (st != MK_OK) return st;
  if (!sc->ready || sc->epoch >= 0x7FFFFFFE) {
    // flags to zero and control words to their reset values, by a fill kernel
    hipError_t e = mk::launch_ws_init(scratch_flags(*sc), (int)mk::kScratchFlags,
                                      scratch_slots(*sc), s);
    if (e != hipSuccess) return hip_fail(e, "clearing the allocation-free workspace");
    sc->ready = true;
    sc->epoch = 0;
  }
  a.P = scratch_partial(*sc);
  a.flags = scratch_flags(*sc);
  a.pub = ar_pub_slots(a, a.flags);
  a.slots = scratch_slots(*sc);
  a.epoch = ++sc->epoch;
  hipError_t e = mk::launch_fused(c.L.shape, peer_dtype, c_dtype, a, s);
  if (e != hipSuccess) return hip_fail(e, "fused kernel launch");
  return MK_OK;
}

// GEMM kernels of the baselines: 256x256 tiles take the in-place kernel's
// eight-wave layout under its option (MK_OPT_STATIC_TILES = 2) when there are
// more tiles than compute units, where it is the faster GEMM (8192 x 8192 x 8192:
// 895-900 us against 919-951 us with four waves, bitwise the same).
int gemm_waves8(const Launch& L, const mk::GemmArgs& g) {
  return L.shape == mk::SHAPE_256 && options().static_tiles == 2 &&
                 (int64_t)g.tiles_m * g.tiles_n > L.info.cus
             ? 1
             : 0;
}

mk_status_t mk_gemm_then_reduce_baseline(const void* A, const void* B, const void* peers,
                                         int n_peers, void* C, int64_t M, int64_t N, int64_t K,
                                         int peer_dtype, int c_dtype, void* stream) {
  mk_status_t st = validate(A, B, peers, n_peers, C, M, N, K, peer_dtype, c_dtype);
  if (st != MK_OK) return st;
  Launch L;
  st = prepare(M, N, K, n_peers, peer_dtype, c_dtype, L);
  if (st != MK_OK) return st;
  if (M == 0 || N == 0) return MK_OK;
  hipStream_t s = (hipStream_t)stream;
  std::lock_guard<std::mutex> lk(g_ws_mu);
  Workspace* w = nullptr;
  const int T = (int)(L.tiles_m * L.tiles_n);
  st = get_ws(L.dev, s, (size_t)(M * N), T, &w);
  if (st != MK_OK) return st;
  mk::GemmArgs g;
  g.A = (const uint16_t*)A;
  g.B = (const uint16_t*)B;
  g.P = w->P;
  g.M = M;
  g.N = N;
  g.K = K;
  g.tiles_m = (int)L.tiles_m;
  g.tiles_n = (int)L.tiles_n;
  const int n_xcd = L.info.cus / 32;  // 32 compute units per XCD on gfx950
  g.n_xcd = n_xcd >= 1 && n_xcd <= mk::kMaxXcd ? n_xcd : 1;
  g.waves8 = gemm_waves8(L, g);
  hipError_t e = mk::launch_gemm(L.shape, g, s);
  if (e != hipSuccess) return hip_fail(e, "gemm kernel launch");
  mk::ReduceArgs r;
  r.P = w->P;
  r.peers = peers;
  r.C = C;
  r.M = M;
  r.N = N;
  r.peer_stride = M * N;
  r.n_peers = n_peers;
  r.pad_ = 0;
  e = mk::launch_reduce(peer_dtype, c_dtype, r, reduce_grid(M * N, L.info.cus), s);
  if (e != hipSuccess) return hip_fail(e, "reduce kernel launch");
  return MK_OK;
}

// CU-masked GEMM and reduce streams of the two-stream schedule for a split of
// `split` compute units to the reduce stream, made on first use and again when
// the split changes. Each 32-unit mask word gives its top split/words bits to
// the reduce stream and the rest to the GEMM stream. Whether the device numbers
// its units XCD by XCD or interleaves them over the XCDs, every XCD then holds
// the same share of each stream (split/words is a multiple of 8, the XCD count).
// Caller holds g_ws_mu.
mk_status_t masked_streams(Workspace* w, int cus, int64_t split) {
  const int words = (cus + 31) / 32;
  if (cus % 32 != 0 || split >= cus || split % (8 * words) != 0)
    return fail(MK_ERR_INVALID_ARG,
                "stream CU split %lld: needs a multiple of %d below %d compute units",
                (long long)split, 8 * words, cus);
  if (w->mask_split == split && w->sg_mask && w->sr_mask) return MK_OK;
  hipError_t e = hipSuccess;
  for (hipStream_t* p : {&w->sg_mask, &w->sr_mask}) {
    if (*p) {
      e = hipStreamSynchronize(*p);  // earlier calls may still run on it
      if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
      (void)hipStreamDestroy(*p);
      *p = nullptr;
    }
  }
  w->mask_split = 0;
  const int per = (int)(split / words);
  std::vector<uint32_t> mg(words), mr(words);
  for (int i = 0; i < words; ++i) {
    mr[i] = per >= 32 ? ~0u : (per == 0 ? 0u : ~0u << (32 - per));
    mg[i] = ~mr[i];
  }
  // default priority, like every stream of the library
  e = hipExtStreamCreateWithCUMask(&w->sg_mask, (uint32_t)words, mg.data());
  if (e != hipSuccess) {
    w->sg_mask = nullptr;
    return hip_fail(e, "CU-masked GEMM stream");
  }
  e = hipExtStreamCreateWithCUMask(&w->sr_mask, (uint32_t)words, mr.data());
  if (e != hipSuccess) {
    w->sr_mask = nullptr;
    return hip_fail(e, "CU-masked reduce stream");
  }
  if (!w->ev_start) {
    e = hipEventCreateWithFlags(&w->ev_start, hipEventDisableTiming);
    if (e != hipSuccess) {
      w->ev_start = nullptr;
      return hip_fail(e, "event");
    }
  }
  w->mask_split = split;
  return MK_OK;
}

mk_status_t mk_gemm_ar_two_stream(const void* A, const void* B, const void* peers, int n_peers,
                                  void* C, int64_t M, int64_t N, int64_t K, int peer_dtype,
                                  int c_dtype, void* stream, int n_chunks) {
  mk_status_t st = validate(A, B, peers, n_peers, C, M, N, K, peer_dtype, c_dtype);
  if (st != MK_OK) return st;
  if (n_chunks < 0 || n_chunks > MK_MAX_CHUNKS)
    return fail(MK_ERR_INVALID_ARG, "n_chunks=%d outside [0, %d]", n_chunks, MK_MAX_CHUNKS);
  Launch L;
  st = prepare(M, N, K, n_peers, peer_dtype, c_dtype, L);
  if (st != MK_OK) return st;
  if (M == 0 || N == 0) return MK_OK;
  hipStream_t s = (hipStream_t)stream;
  std::lock_guard<std::mutex> lk(g_ws_mu);
  Workspace* w = nullptr;
  const int T = (int)(L.tiles_m * L.tiles_n);
  st = get_ws(L.dev, s, (size_t)(M * N), T, &w);
  if (st != MK_OK) return st;
  if (!w->s2) {
    // default priority, like every stream of the library
    hipError_t e = hipStreamCreateWithFlags(&w->s2, hipStreamNonBlocking);
    if (e != hipSuccess) {
      w->s2 = nullptr;
      return hip_fail(e, "reduce stream");
    }
    for (hipEvent_t& ev : w->ev) {
      e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
      if (e != hipSuccess) {
        ev = nullptr;
        return hip_fail(e, "event");
      }
    }
  }
  // GEMM kernels on sg, reduce kernels on sr: the caller's stream and the
  // library's second stream, or two CU-masked streams of the library, the GEMM
  // one ordered after everything already on the caller's stream.
  hipStream_t sg = s, sr = w->s2;
  const int64_t split = options().stream_cu_split;
  if (split > 0) {
    st = masked_streams(w, L.info.cus, split);
    if (st != MK_OK) return st;
    hipError_t e0 = hipEventRecord(w->ev_start, s);
    if (e0 == hipSuccess) e0 = hipStreamWaitEvent(w->sg_mask, w->ev_start, 0);
    if (e0 != hipSuccess) return hip_fail(e0, "two-stream schedule");
    sg = w->sg_mask;
    sr = w->sr_mask;
  }
  // Chunks of whole tile rows: chunk i is tile rows [i*tm/c, (i+1)*tm/c).
  const int tm = (int)L.tiles_m;
  int c = n_chunks == 0 ? 4 : n_chunks;
  if (c > tm) c = tm;
  const int BM = mk::shape_bm(L.shape);
  const int n_xcd = L.info.cus / 32;
  hipEvent_t* ev = w->ev;
  // Every reduce waits for an event recorded on the GEMM stream after its
  // chunk's GEMM, hence after all earlier work on the caller's stream (the
  // previous call's reduces included, see the end).
  hipError_t e = hipSuccess;
  for (int i = 0; i < c && e == hipSuccess; ++i) {
    const int64_t r0 = (int64_t)(i * (int64_t)tm / c) * BM;
    int64_t r1 = (int64_t)((i + 1) * (int64_t)tm / c) * BM;
    if (r1 > M) r1 = M;
    mk::GemmArgs g;
    g.A = (const uint16_t*)A + r0 * K;
    g.B = (const uint16_t*)B;
    g.P = w->P + r0 * N;
    g.M = r1 - r0;
    g.N = N;
    g.K = K;
    g.tiles_m = (int)((r1 - r0 + BM - 1) / BM);
    g.tiles_n = (int)L.tiles_n;
    g.n_xcd = n_xcd >= 1 && n_xcd <= mk::kMaxXcd ? n_xcd : 1;
    g.waves8 = gemm_waves8(L, g);
    e = mk::launch_gemm(L.shape, g, sg);
    if (e != hipSuccess) break;
    // the chunk's partial rows are complete when the GEMM kernel ends
    e = hipEventRecord(ev[i], sg);
    if (e == hipSuccess) e = hipStreamWaitEvent(sr, ev[i], 0);
    if (e != hipSuccess) break;
    mk::ReduceArgs r;
    r.P = w->P + r0 * N;
    r.peers = (const char*)peers + (size_t)(r0 * N) * dt_size(peer_dtype);
    r.C = (char*)C + (size_t)(r0 * N) * dt_size(c_dtype);
    r.M = r1 - r0;
    r.N = N;
    r.peer_stride = M * N;
    r.n_peers = n_peers;
    r.pad_ = 0;
    e = mk::launch_reduce(peer_dtype, c_dtype, r, reduce_grid(r.M * N, L.info.cus), sr);
  }
  // the call ends on the caller's stream when the last reduce has finished
  // (which waited for the last GEMM)
  if (e == hipSuccess) e = hipEventRecord(ev[c], sr);
  if (e == hipSuccess) e = hipStreamWaitEvent(s, ev[c], 0);
  if (e != hipSuccess) return hip_fail(e, "two-stream schedule");
  return MK_OK;
}

mk_status_t mk_gemm_rs_local(const void* A, const void* B, const void* peers, int n_peers, void* C,
                             void* send, int64_t M, int64_t N, int64_t K, int64_t own_m0,
                             int64_t own_m1, int peer_dtype, int c_dtype, void* stream,
                             int n_reduce_wg) {
  mk_status_t st = validate_rs(A, B, peers, n_peers, C, send, M, N, K, own_m0, own_m1, peer_dtype,
                               c_dtype);
  if (st != MK_OK) return st;
  if (n_reduce_wg < MK_ADAPTIVE) return fail(MK_ERR_INVALID_ARG, "n_reduce_wg=%d", n_reduce_wg);
  Launch L;
  st = prepare(M, N, K, n_peers, peer_dtype, c_dtype, L, false);
  if (st != MK_OK) return st;
  const int G = rs_grid_size(L, peer_dtype, c_dtype);
  if (n_reduce_wg > G - 1)
    return fail(MK_ERR_INVALID_ARG, "n_reduce_wg=%d outside [0, %d]", n_reduce_wg, G - 1);
  if (M == 0 || N == 0) return MK_OK;
  hipStream_t s = (hipStream_t)stream;
  const Options opt = options();
  std::lock_guard<std::mutex> lk(g_ws_mu);
  Workspace* w = nullptr;
  const int T = (int)(L.tiles_m * L.tiles_n);
  st = get_ws(L.dev, s, (size_t)(M * N), T, &w);
  if (st != MK_OK) return st;
  if (++w->epoch >= 0x7FFFFFFF) {
    hipError_t e = mk::launch_ws_init(w->flags, w->flags_cap, nullptr, s);
    if (e != hipSuccess) return hip_fail(e, "flag reset");
    w->epoch = 1;
  }
  mk::FusedArgs a;
  memset(&a, 0, sizeof a);
  a.A = (const uint16_t*)A;
  a.B = (const uint16_t*)B;
  a.peers = peers;
  a.C = C;
  a.P = w->P;
  a.flags = w->flags;
  a.slots = w->slots;
  a.tel = nullptr;
  a.M = M;
  a.N = N;
  a.K = K;
  a.n_peers = n_peers;
  a.tiles_m = (int)L.tiles_m;
  a.tiles_n = (int)L.tiles_n;
  a.T = T;
  a.G = G;
  a.epoch = w->epoch;
  a.ctrl_period = opt.ctrl_period < 1 ? 1 : (int)opt.ctrl_period;
  a.withhold_tile = (int)opt.withhold_tile;
  a.spin_limit = (unsigned long long)(opt.spin_timeout_us < 1 ? 1 : opt.spin_timeout_us) * 100ull;
  mk::queue_plan(L.info.cus, G, (int)opt.flag_scope, a.n_xcd, a.flag_scope);
  a.shared_lines = N % 32 != 0 ? 1 : 0;  // partial rows not whole 128-byte lines
  a.early = 0;
  a.rs = 1;
  // Tile rows that hold owned rows are handed to reducers (their reduce is the
  // heavy part and spreads over 64-row units); every other tile is computed and
  // published in place. They lead each XCD's queue.
  const int BM = mk::shape_bm(L.shape);
  a.tmo0 = (int)(own_m0 / BM);
  a.tmo1 = own_m1 > own_m0 ? (int)((own_m1 + BM - 1) / BM) : a.tmo0;
  a.own0 = own_m0;
  a.own1 = own_m1;
  a.send = send;
  a.n_inplace = 0;  // not used by a ReduceScatter share
  a.T_r = (a.tmo1 - a.tmo0) * a.tiles_n;
  // Controller: the handed-over tiles' reduce against the GEMM and the publish
  // stores, both at roofline speed; at most the reducers that saturate HBM.
  {
    const int occ = L.shape == mk::SHAPE_256 ? 1 : 2;
    int cap = (int)ceil(5.5e12 / 40e9) * occ;
    cap = (cap + a.n_xcd - 1) / a.n_xcd * a.n_xcd;
    a.reducer_cap = opt.reducer_cap > 0 ? (int)opt.reducer_cap : (cap < G - 1 ? cap : G - 1);
    // As for the AllReduce share: with tiles handled in place, a dedicated
    // reducer takes a compute unit from the GEMM (on the 4096x8192x1792 shape one
    // reducer per XCD leaves a third round of tiles: 175 -> 211 us); the derived
    // cap is then zero and every workgroup drains the handed-over units.
    if (opt.reducer_cap <= 0 && a.T_r < a.T && !a.dyn) a.reducer_cap = 0;
    const double rows_h = (double)(a.tmo1 - a.tmo0) * BM;
    const double own = (double)(own_m1 - own_m0);
    const double t_r = (rows_h * N * 4.0 + own * N * (n_peers * (double)dt_size(peer_dtype) +
                        dt_size(c_dtype)) + (rows_h - own) * N * dt_size(peer_dtype)) / 8.0e12;
    const double t_c = 2.0 * M * N * K / 2.5e15 + ((double)M - rows_h) * N * dt_size(peer_dtype) / 8.0e12;
    a.seed_x = t_r + t_c > 0 ? (float)(t_r / (t_r + t_c)) : 0.0f;
  }
  if (n_reduce_wg == MK_ADAPTIVE) {
    a.adaptive = 1;
    int it = (int)(a.seed_x * G + 0.5f);
    it = it < 0 ? 0 : (it > a.reducer_cap ? a.reducer_cap : it);
    a.init_target = it;
  } else {
    a.adaptive = 0;
    a.init_target = n_reduce_wg;
  }
  hipError_t e = mk::launch_fused(L.shape, peer_dtype, c_dtype, a, s);
  if (e != hipSuccess) return hip_fail(e, "fused kernel launch");
  return MK_OK;
}

mk_status_t mk_gemm_rs_baseline(const void* A, const void* B, const void* peers, int n_peers,
                                void* C, void* send, int64_t M, int64_t N, int64_t K,
                                int64_t own_m0, int64_t own_m1, int peer_dtype, int c_dtype,
                                void* stream) {
  mk_status_t st = validate_rs(A, B, peers, n_peers, C, send, M, N, K, own_m0, own_m1, peer_dtype,
                               c_dtype);
  if (st != MK_OK) return st;
  Launch L;
  st = prepare(M, N, K, n_peers, peer_dtype, c_dtype, L, false);
  if (st != MK_OK) return st;
  if (M == 0 || N == 0) return MK_OK;
  hipStream_t s = (hipStream_t)stream;
  std::lock_guard<std::mutex> lk(g_ws_mu);
  Workspace* w = nullptr;
  const int T = (int)(L.tiles_m * L.tiles_n);
  st = get_ws(L.dev, s, (size_t)(M * N), T, &w);
  if (st != MK_OK) return st;
  mk::GemmArgs g;
  g.A = (const uint16_t*)A;
  g.B = (const uint16_t*)B;
  g.P = w->P;
  g.M = M;
  g.N = N;
  g.K = K;
  g.tiles_m = (int)L.tiles_m;
  g.tiles_n = (int)L.tiles_n;
  const int n_xcd = L.info.cus / 32;
  g.n_xcd = n_xcd >= 1 && n_xcd <= mk::kMaxXcd ? n_xcd : 1;
  g.waves8 = gemm_waves8(L, g);
  hipError_t e = mk::launch_gemm(L.shape, g, s);
  if (e != hipSuccess) return hip_fail(e, "gemm kernel launch");
  const int64_t own = own_m1 - own_m0;
  // owned rows: the reduce kernel; the other rows: the same kernel without
  // peers, which rounds the partial to the peer type
  const int64_t r0[3] = {own_m0, 0, own_m1}, r1[3] = {own_m1, own_m0, M};
  for (int part = 0; part < 3; ++part) {
    const int64_t rows = r1[part] - r0[part];
    if (rows <= 0) continue;
    mk::ReduceArgs r;
    r.P = w->P + r0[part] * N;
    r.M = rows;
    r.N = N;
    r.pad_ = 0;
    if (part == 0) {
      r.peers = peers;
      r.C = C;
      r.peer_stride = own * N;
      r.n_peers = n_peers;
      e = mk::launch_reduce(peer_dtype, c_dtype, r, reduce_grid(rows * N, L.info.cus), s);
    } else {
      r.peers = nullptr;
      r.C = (char*)send + (size_t)(r0[part] * N) * dt_size(peer_dtype);
      r.peer_stride = 0;
      r.n_peers = 0;
      e = mk::launch_reduce(peer_dtype, peer_dtype, r, reduce_grid(rows * N, L.info.cus), s);
    }
    if (e != hipSuccess) return hip_fail(e, "reduce kernel launch");
  }
  return MK_OK;
}

mk_status_t mk_gemm_ag_local(const void* A_local, const void* peers_A, int n_peers, void* A_full,
                             const void* B, void* C, int64_t Ms, int64_t N, int64_t K, int rank,
                             int c_dtype, void* stream, int n_comm_wg) {
  mk_status_t st = validate_ag(A_local, peers_A, n_peers, A_full, B, C, Ms, N, K, rank, c_dtype);
  if (st != MK_OK) return st;
  if (n_comm_wg < MK_ADAPTIVE) return fail(MK_ERR_INVALID_ARG, "n_comm_wg=%d", n_comm_wg);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MK_ERR_NO_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  DeviceInfo info;
  st = device_info(dev, info);
  if (st != MK_OK) return st;
  const int P = n_peers + 1;
  const int shape = ag_shape(Ms, P, N, info.cus);
  const int BM = mk::shape_bm(shape), BN = mk::shape_bn(shape);
  const int64_t M = (int64_t)P * Ms;
  const int64_t NB = M / BM, tiles_n = (N + BN - 1) / BN;
  if (NB * tiles_n > (1 << 30) || NB * mk::kAgMaxPieces > (1 << 30))
    return fail(MK_ERR_UNSUPPORTED, "too many tiles");
  const int G = ag_grid_size(info, shape, c_dtype, NB * tiles_n);
  if (n_comm_wg > G - 1)
    return fail(MK_ERR_INVALID_ARG, "n_comm_wg=%d outside [0, %d]", n_comm_wg, G - 1);
  if (M == 0) return MK_OK;
  hipStream_t s = (hipStream_t)stream;
  const Options opt = options();
  std::lock_guard<std::mutex> lk(g_ws_mu);
  Workspace* w = nullptr;
  st = get_ws(dev, s, 0, 0, &w);
  if (st != MK_OK) return st;
  const int64_t n_flags = NB * mk::kAgMaxPieces;
  if (n_flags > w->ag_cap) {
    e = hipStreamSynchronize(s);  // earlier calls on this stream may still use the old flags
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    if (w->ag_landed) (void)hipFree(w->ag_landed);
    w->ag_landed = nullptr;
    w->ag_cap = 0;
    const int cap = n_flags < 4096 ? 4096 : (int)n_flags;
    e = hipMalloc(&w->ag_landed, sizeof(int) * (size_t)cap);
    if (e != hipSuccess) return fail(MK_ERR_WORKSPACE, "piece flags: %s", hipGetErrorString(e));
    e = mk::launch_ws_init(w->ag_landed, cap, nullptr, s);
    if (e != hipSuccess) return hip_fail(e, "piece flag init");
    w->ag_cap = cap;
  }
  // Pieces: at most kAgMaxPieces per band, each a whole number of 64-column
  // steps (the deepest k-tile), so that a k-tile never waits for two pieces. A
  // tile may read a piece while the next ones are still landing only if no
  // 128-byte line holds bytes of two pieces: A_full 128-byte aligned, rows and
  // piece widths multiples of 64 columns. Otherwise a tile waits for every piece
  // of its band.
  const int64_t kt_total = (K + 31) / 32;
  int64_t ktpp = (kt_total + 7) / 8;  // about eight pieces per band
  const bool lines_ok = ((uintptr_t)A_full) % 128 == 0 && K % 64 == 0;
  if (ktpp % 2 == 1) ktpp += 1;
  mk::AgArgs a;
  memset(&a, 0, sizeof a);
  a.A_local = (const uint16_t*)A_local;
  a.peers = (const uint16_t*)peers_A;
  a.A_full = (uint16_t*)A_full;
  a.B = (const uint16_t*)B;
  a.C = C;
  a.landed = w->ag_landed;
  a.slots = w->slots;
  a.M = M;
  a.N = N;
  a.K = K;
  a.Ms = Ms;
  a.KP = ktpp * 32;
  a.P = P;
  a.rank = rank;
  a.bps = (int)(Ms / BM);
  a.NB = (int)NB;
  a.ktpp = ktpp > 0 ? (int)ktpp : 1;
  a.npc = K > 0 ? (int)((K + a.KP - 1) / a.KP) : 0;
  a.inloop = lines_ok ? 1 : 0;
  a.tiles_n = (int)tiles_n;
  a.T = (int)(NB * tiles_n);
  a.G = G;
  // bands are owned per XCD where the device's layout allows it (queue_plan)
  mk::queue_plan(info.cus, G, (int)opt.flag_scope, a.n_xcd, a.flag_scope);
  // Default: four landing workgroups per XCD (the grid's workgroups beyond the
  // tiles when it has room); the others land pieces only while the first piece
  // of their tile's band is missing.
  a.n_comm = n_comm_wg >= 0 ? n_comm_wg : (4 * a.n_xcd < G ? 4 * a.n_xcd : G - 1);
  a.spin_limit = (unsigned long long)(opt.spin_timeout_us < 1 ? 1 : opt.spin_timeout_us) * 100ull;
  e = mk::launch_ag(shape, c_dtype, a, s);
  if (e != hipSuccess) return hip_fail(e, "AllGather+GEMM kernel launch");
  return MK_OK;
}

mk_status_t mk_gemm_ag_baseline(const void* A_local, const void* peers_A, int n_peers,
                                void* A_full, const void* B, void* C, int64_t Ms, int64_t N,
                                int64_t K, int rank, int c_dtype, void* stream) {
  mk_status_t st = validate_ag(A_local, peers_A, n_peers, A_full, B, C, Ms, N, K, rank, c_dtype);
  if (st != MK_OK) return st;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MK_ERR_NO_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  DeviceInfo info;
  st = device_info(dev, info);
  if (st != MK_OK) return st;
  const int P = n_peers + 1;
  const int64_t M = (int64_t)P * Ms;
  if (M == 0) return MK_OK;
  hipStream_t s = (hipStream_t)stream;
  if (K > 0) {
    mk::AgCopyArgs c;
    c.A_local = (const uint16_t*)A_local;
    c.peers = (const uint16_t*)peers_A;
    c.A_full = (uint16_t*)A_full;
    c.Ms = Ms;
    c.K = K;
    c.P = P;
    c.rank = rank;
    e = mk::launch_ag_copy(c, copy_grid(M * K, info.cus), s);
    if (e != hipSuccess) return hip_fail(e, "gather kernel launch");
  }
  if (N == 0) return MK_OK;
  const int shape = ag_shape(Ms, P, N, info.cus);
  mk::GemmArgs g;
  g.A = (const uint16_t*)A_full;
  g.B = (const uint16_t*)B;
  g.P = nullptr;
  g.M = M;
  g.N = N;
  g.K = K;
  g.tiles_m = (int)(M / mk::shape_bm(shape));
  g.tiles_n = (int)((N + mk::shape_bn(shape) - 1) / mk::shape_bn(shape));
  const int n_xcd = info.cus / 32;
  g.n_xcd = n_xcd >= 1 && n_xcd <= mk::kMaxXcd ? n_xcd : 1;
  g.waves8 = 0;
  e = mk::launch_gemm_c(shape, c_dtype, g, C, s);
  if (e != hipSuccess) return hip_fail(e, "GEMM kernel launch");
  return MK_OK;
}

int mk_ag_grid(int64_t Ms, int n_peers, int64_t N, int64_t K, int c_dtype) {
  (void)K;
  if (c_dtype != MK_DT_BF16 && c_dtype != MK_DT_F32) return -(int)MK_ERR_INVALID_ARG;
  if (Ms < 0 || N < 0 || n_peers < 0 || n_peers > MK_MAX_PEERS || Ms % 128 != 0)
    return -(int)MK_ERR_INVALID_ARG;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -(int)MK_ERR_NO_DEVICE;
  DeviceInfo info;
  mk_status_t st = device_info(dev, info);
  if (st != MK_OK) return -(int)st;
  const int P = n_peers + 1;
  const int shape = ag_shape(Ms, P, N, info.cus);
  const int64_t NB = (int64_t)P * Ms / mk::shape_bm(shape);
  const int64_t tiles_n = (N + mk::shape_bn(shape) - 1) / mk::shape_bn(shape);
  return ag_grid_size(info, shape, c_dtype, NB * tiles_n);
}

mk_status_t mk_flag_handoff(int iters, int flag_scope, int cross_xcd, void* stream, void* out) {
  if (iters < 1 || iters > (1 << 24)) return fail(MK_ERR_INVALID_ARG, "iters=%d outside [1, 2^24]", iters);
  if (flag_scope < 0 || flag_scope > 2) return fail(MK_ERR_INVALID_ARG, "flag_scope=%d", flag_scope);
  if (cross_xcd != 0 && cross_xcd != 1) return fail(MK_ERR_INVALID_ARG, "cross_xcd=%d", cross_xcd);
  if (!out || ((uintptr_t)out) % 16 != 0) return fail(MK_ERR_INVALID_ARG, "out is NULL or not 16-byte aligned");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MK_ERR_NO_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  DeviceInfo info;
  mk_status_t st = device_info(dev, info);
  if (st != MK_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  const Options opt = options();
  std::lock_guard<std::mutex> lk(g_ws_mu);
  Workspace* w = nullptr;
  st = get_ws(dev, s, 0, 0, &w);
  if (st != MK_OK) return st;
  const unsigned call = (unsigned)(++w->handoffs);
  e = hipMemsetAsync(out, 0, 5 * sizeof(unsigned long long), s);
  if (e != hipSuccess) return hip_fail(e, "clearing out");
  const unsigned long long limit =
      (unsigned long long)(opt.spin_timeout_us < 1 ? 1 : opt.spin_timeout_us) * 100ull;
  e = mk::launch_pingpong(w->slots, call, iters, flag_scope, cross_xcd, limit,
                          (unsigned long long*)out, s);
  if (e != hipSuccess) return hip_fail(e, "hand-off kernel launch");
  return MK_OK;
}

mk_status_t mk_mfma_peak(int iters, int n_workgroups, void* out, void* stream) {
  if (iters < 1 || iters > (1 << 24)) return fail(MK_ERR_INVALID_ARG, "iters=%d outside [1, 2^24]", iters);
  if (n_workgroups < 1 || n_workgroups > (1 << 16))
    return fail(MK_ERR_INVALID_ARG, "n_workgroups=%d outside [1, 65536]", n_workgroups);
  if (!out || ((uintptr_t)out) % 4 != 0) return fail(MK_ERR_INVALID_ARG, "out is NULL or not 4-byte aligned");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MK_ERR_NO_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  e = mk::launch_mfma_peak(iters, n_workgroups, (float*)out, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "matrix-core peak kernel launch");
  return MK_OK;
}

mk_status_t mk_stream_status(void* stream) {
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  int dev = 0;
  e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  // the error words of the stream's workspace and of the device's
  // allocation-free workspace (if calls used it)
  unsigned long long* slots[2] = {nullptr, nullptr};
  {
    std::lock_guard<std::mutex> lk(g_ws_mu);
    auto it = g_ws.find(std::make_pair(dev, s));
    if (it != g_ws.end()) slots[0] = it->second->slots;
  }
  {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    auto it = g_scratch.find(dev);
    if (it != g_scratch.end() && it->second.ready) slots[1] = scratch_slots(it->second);
  }
  for (unsigned long long* sl : slots) {
    if (!sl) continue;
    unsigned long long word = 0;
    e = hipMemcpy(&word, sl + (size_t)mk::S_ERROR * mk::kSlotWords, sizeof word,
                  hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "reading the device error word");
    if (word == 0) continue;
    e = mk::launch_clear_error(sl, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "clearing the device error word");
    int code = (int)(word & 0xFFFFFFFFu);
    return fail((mk_status_t)code, "device reported error %d (%s)", code, mk_status_string(code));
  }
  return MK_OK;
}

mk_status_t mk_workspace_reset(int device) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  e = hipSetDevice(device);
  if (e != hipSuccess) return fail(MK_ERR_NO_DEVICE, "hipSetDevice(%d): %s", device, hipGetErrorString(e));
  e = hipDeviceSynchronize();
  std::lock_guard<std::mutex> lk(g_ws_mu);
  for (auto it = g_ws.begin(); it != g_ws.end();) {
    if (it->first.first == device) {
      free_ws(it->second);
      it = g_ws.erase(it);
    } else {
      ++it;
    }
  }
  (void)hipSetDevice(cur);
  {
    std::lock_guard<std::mutex> lk2(g_scratch_mu);
    auto it = g_scratch.find(device);
    if (it != g_scratch.end()) it->second.ready = false;  // cleared again on next use
  }
  if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
  return MK_OK;
}

int mk_queue_plan(int cus, int grid, int flag_scope, int* n_xcd) {
  if (cus < 1 || grid < 1 || (flag_scope != 0 && flag_scope != 1) || !n_xcd)
    return -(int)MK_ERR_INVALID_ARG;
  int scope = 1;
  mk::queue_plan(cus, grid, flag_scope, *n_xcd, scope);
  return scope;
}

int mk_num_workgroups(int device) {
  DeviceInfo d;
  mk_status_t st = device_info(device, d);
  if (st != MK_OK) return -(int)st;
  return d.cus * d.occ[mk::SHAPE_256][MK_DT_BF16][MK_DT_BF16];
}

int mk_fused_grid(int64_t M, int64_t N, int64_t K, int n_peers, int peer_dtype, int c_dtype) {
  if (peer_dtype != MK_DT_BF16 && peer_dtype != MK_DT_F32) return -(int)MK_ERR_INVALID_ARG;
  if (c_dtype != MK_DT_BF16 && c_dtype != MK_DT_F32) return -(int)MK_ERR_INVALID_ARG;
  if (M < 0 || N < 0 || K < 0 || n_peers < 0) return -(int)MK_ERR_INVALID_ARG;
  Launch L;
  mk_status_t st =
      prepare(M, N, K, n_peers, peer_dtype, c_dtype, L, true, true, ws_auto_allowed(MK_ADAPTIVE));
  if (st != MK_OK) return -(int)st;
  return fused_grid_size(L, n_peers, peer_dtype, c_dtype);
}

int mk_fused_schedule(int64_t M, int64_t N, int64_t K, int n_peers, int peer_dtype, int c_dtype) {
  if (peer_dtype != MK_DT_BF16 && peer_dtype != MK_DT_F32) return -(int)MK_ERR_INVALID_ARG;
  if (c_dtype != MK_DT_BF16 && c_dtype != MK_DT_F32) return -(int)MK_ERR_INVALID_ARG;
  if (M < 0 || N < 0 || K < 0 || n_peers < 0) return -(int)MK_ERR_INVALID_ARG;
  Launch L;
  mk_status_t st =
      prepare(M, N, K, n_peers, peer_dtype, c_dtype, L, true, true, ws_auto_allowed(MK_ADAPTIVE));
  if (st != MK_OK) return -(int)st;
  return L.shape;
}

mk_status_t mk_set_option(int option, int64_t value) {
  std::lock_guard<std::mutex> lk(g_opt_mu);
  switch (option) {
    case MK_OPT_SPIN_TIMEOUT_US:
      if (value < 1) return fail(MK_ERR_INVALID_ARG, "spin timeout must be >= 1 us");
      g_opt.spin_timeout_us = value;
      return MK_OK;
    case MK_OPT_WITHHOLD_TILE:
      g_opt.withhold_tile = value < 0 ? -1 : value;
      return MK_OK;
    case MK_OPT_CTRL_PERIOD:
      if (value < 1) return fail(MK_ERR_INVALID_ARG, "controller period must be >= 1");
      g_opt.ctrl_period = value;
      return MK_OK;
    case MK_OPT_TILE_SHAPE:
      if (value < 0 || value > 5) return fail(MK_ERR_INVALID_ARG, "tile shape %lld", (long long)value);
      g_opt.tile_shape = value;
      return MK_OK;
    case MK_OPT_FLAG_SCOPE:
      if (value < 0 || value > 1) return fail(MK_ERR_INVALID_ARG, "flag scope %lld", (long long)value);
      g_opt.flag_scope = value;
      return MK_OK;
    case MK_OPT_REDUCER_CAP:
      if (value < 0) return fail(MK_ERR_INVALID_ARG, "reducer cap %lld", (long long)value);
      g_opt.reducer_cap = value;
      return MK_OK;
    case MK_OPT_INPLACE:
      if (value < -2 || value > (1 << 30)) return fail(MK_ERR_INVALID_ARG, "in-place tiles %lld", (long long)value);
      g_opt.inplace = value;
      return MK_OK;
    case MK_OPT_EARLY:
      if (value < -1 || value > 1) return fail(MK_ERR_INVALID_ARG, "early reduce %lld", (long long)value);
      g_opt.early = value;
      return MK_OK;
    case MK_OPT_KSPLIT:
      if (value != -1 && value != 1 && value != 2)
        return fail(MK_ERR_INVALID_ARG, "k-split %lld", (long long)value);
      g_opt.ksplit = value;
      return MK_OK;
    case MK_OPT_STREAM_CU_SPLIT:
      // the device-dependent checks happen at the call
      if (value < 0 || value > 4096 || value % 8 != 0)
        return fail(MK_ERR_INVALID_ARG, "stream CU split %lld", (long long)value);
      g_opt.stream_cu_split = value;
      return MK_OK;
    case MK_OPT_STATIC_TILES:
      if (value < 0 || value > 2) return fail(MK_ERR_INVALID_ARG, "static tiles %lld", (long long)value);
      g_opt.static_tiles = value;
      return MK_OK;
  }
  return fail(MK_ERR_INVALID_ARG, "unknown option %d", option);
}

int64_t mk_get_option(int option) {
  std::lock_guard<std::mutex> lk(g_opt_mu);
  switch (option) {
    case MK_OPT_SPIN_TIMEOUT_US: return g_opt.spin_timeout_us;
    case MK_OPT_WITHHOLD_TILE: return g_opt.withhold_tile;
    case MK_OPT_CTRL_PERIOD: return g_opt.ctrl_period;
    case MK_OPT_TILE_SHAPE: return g_opt.tile_shape;
    case MK_OPT_FLAG_SCOPE: return g_opt.flag_scope;
    case MK_OPT_REDUCER_CAP: return g_opt.reducer_cap;
    case MK_OPT_INPLACE: return g_opt.inplace;
    case MK_OPT_EARLY: return g_opt.early;
    case MK_OPT_KSPLIT: return g_opt.ksplit;
    case MK_OPT_STREAM_CU_SPLIT: return g_opt.stream_cu_split;
    case MK_OPT_STATIC_TILES: return g_opt.static_tiles;
  }
  return -1;
}

int mk_controller_eval(int G, int T, int T_r, int computed, int reduced, uint64_t busy_c,
                       uint64_t busy_r, float seed_x, int current, int cap) {
  return mk::controller_rule(G, T, T_r, computed, reduced, busy_c, busy_r, seed_x, current, cap);
}

const char* mk_status_string(int status) {
  switch (status) {
    case MK_OK: return "MK_OK";
    case MK_ERR_INVALID_ARG: return "MK_ERR_INVALID_ARG";
    case MK_ERR_UNSUPPORTED: return "MK_ERR_UNSUPPORTED";
    case MK_ERR_HIP: return "MK_ERR_HIP";
    case MK_ERR_TIMEOUT: return "MK_ERR_TIMEOUT";
    case MK_ERR_NO_DEVICE: return "MK_ERR_NO_DEVICE";
    case MK_ERR_WORKSPACE: return "MK_ERR_WORKSPACE";
    case MK_ERR_INTERNAL: return "MK_ERR_INTERNAL";
  }
  return "MK_ERR_UNKNOWN";
}

const char* mk_last_error(void) { return g_last_error.c_str(); }

int mk_version(void) { return 1; }

}  // extern "C"
