// mk_controller.h -- the reducer-count rule run by the on-GPU controller.
//
// The pages say what the controller does, not how: it reads progress counters
// and publishes a target number of communication blocks (thelatestinai.com
// page, Figure 2 caption), it adapts the split from measured progress, and for
// GEMM+AllReduce its target moves towards communication as the computation
// nears completion (Figure 7a). The rule's own formula is not recoverable from
// the pages, so this file states the rule adopted here:
//
//   remaining compute work   W_c = (T - c) / rho_c   (workgroup-time)
//   remaining reduce work    W_r = (T_r - r) / rho_r
//   reducer share            x   = W_r / (W_c + W_r)
//   target                   clamp(round(G * x), 1, G - 1) while compute remains,
//                            G once every tile is computed.
//
// T_r <= T is the number of tiles handed to reducers (the others are reduced in
// place by the workgroup that computed them, and their whole time counts as
// compute). rho_c = tiles computed per unit of compute-role busy time; rho_r =
// handed-over tiles reduced per unit of reducer busy time *excluding* time
// spent waiting for flags, so idle reducers do not look slow. Both finish at the same time when
// the reducers hold the share x of the workgroups. Until both rates have been
// measured, x is the host's seed (roofline estimate). A change smaller than
// max(1, G/64) is ignored (hysteresis).
//
// The reduce is a stream from HBM: past the number of reducers that saturates
// HBM bandwidth (`cap`), more reducers do not reduce faster, they only take
// compute units away from the GEMM, and the per-workgroup rate rho_r that the
// rule sees drops because the stream is shared. While compute remains the
// target is therefore limited to `cap` (the host derives it from HBM bandwidth
// over one reducer workgroup's streaming rate).
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define MK_HD __host__ __device__
#else
#define MK_HD
#endif

namespace mk {

MK_HD inline int controller_rule(int G, int T, int T_r, int computed, int reduced,
                                 uint64_t busy_c, uint64_t busy_r, float seed_x, int current,
                                 int cap) {
  if (G <= 1) return G <= 0 ? 0 : current;
  if (computed >= T) return G;
  float x = seed_x;
  if (reduced >= T_r) {
    x = 0.0f;  // nothing left for reducers while compute remains
  } else if (computed > 0 && reduced > 0 && busy_c > 0 && busy_r > 0) {
    // W = remaining / rate = remaining * busy / done
    float wc = (float)(T - computed) * ((float)busy_c / (float)computed);
    float wr = (float)(T_r - reduced) * ((float)busy_r / (float)reduced);
    x = (wc + wr) > 0.0f ? wr / (wc + wr) : seed_x;
  }
  if (!(x >= 0.0f)) x = 0.0f;  // also catches NaN
  if (x > 1.0f) x = 1.0f;
  int target = (int)(x * (float)G + 0.5f);
  // cap < 0: up to G-1 reducers; cap == 0: none while compute remains
  const int hi = cap >= 0 && cap < G - 1 ? cap : G - 1;
  const int lo = hi < 1 ? hi : 1;
  if (target > hi) target = hi;
  if (target < lo) target = lo;
  int band = G / 64 > 1 ? G / 64 : 1;
  int d = target - current;
  if (d < 0) d = -d;
  if (current >= lo && current <= hi && d < band) return current;
  return target;
}

}  // namespace mk
