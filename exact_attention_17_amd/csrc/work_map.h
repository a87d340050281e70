// Workgroup -> (batch, query head, query tile) order shared by the forward
// kernel and the dQ kernel of the backward pass, dense and varlen.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

struct WorkItem {
  int b, h, qt;
  int q_base, k_base;   // first token of the sequence (varlen) or 0
  int Lq, Lk;
  bool valid;
};

// Dense work order.  Blocks are dealt to the 8 XCDs round-robin (block id % 8),
// so when the KV-group count (B * Hkv) is a multiple of 8, XCD x gets KV groups
// x, x+8, ...  Within an XCD the groups are taken in chunks of `chunk_groups`
// (sized so a chunk's workgroups about fill the XCD), and inside a chunk the
// query tiles go heaviest (latest causal rows) first.  A chunk's K/V then
// stays in the XCD's L2 while all its query tiles stream through it.
template <class Params>
__device__ __forceinline__ WorkItem map_work_dense(const Params& p, int id) {
  WorkItem w;
  if (p.xcd_groups > 0) {
    const int x = id & 7, s = id >> 3;
    const int A = p.xcd_groups >> 3;                   // KV groups per XCD
    const int per_group = p.group * p.num_q_tiles;     // workgroups per KV group
    const int chunk = s / (p.chunk_groups * per_group);
    const int c0 = chunk * p.chunk_groups;
    const int cn = min(p.chunk_groups, A - c0);        // groups in this chunk
    const int sl = s - c0 * per_group;
    const int qrev = sl / (cn * p.group), r = sl - qrev * (cn * p.group);
    const int gl = c0 + r / p.group, gq = r % p.group;
    const int kvg = x + 8 * gl;
    w.b = kvg / p.Hkv;
    w.h = (kvg - w.b * p.Hkv) * p.group + gq;
    w.qt = p.num_q_tiles - 1 - qrev;
  } else {
    const int NH = p.B * p.Hq;
    const int qrev = id / NH, r = id - qrev * NH;
    w.b = r / p.Hq;
    w.h = r - w.b * p.Hq;
    w.qt = p.num_q_tiles - 1 - qrev;
  }
  w.q_base = 0;
  w.k_base = 0;
  w.Lq = p.Lq;
  w.Lk = p.Lk;
  w.valid = true;
  return w;
}

// Varlen: without a plan, tile slots of sequence b start at
// T_b = floor(cu_q[b] / 128) + b, which leaves room for its ceil(len_b / 128)
// tiles before T_{b+1}; with a plan, slot t is the plan's item t.
template <class Params>
__device__ __forceinline__ WorkItem map_work_varlen(const Params& p, int id) {
  WorkItem w;
  const int r = id % p.Hq, t = id / p.Hq;
  if (p.xcd_groups > 0) {
    const int x = r & 7, i = r >> 3;
    const int kvh = x + 8 * (i / p.group);
    w.h = kvh * p.group + (i % p.group);
  } else {
    w.h = r;
  }
  if (p.plan) {
    // planned run: item t of the host plan names (sequence, query tile); the
    // plan is uniform per workgroup, so read it through the scalar cache
    const __attribute__((address_space(4))) int* pc =
        (const __attribute__((address_space(4))) int*)p.plan;
    const int b = pc[2 * t], qt = pc[2 * t + 1];
    w.valid = b >= 0 && b < p.B;
    if (!w.valid) return w;
    w.b = b;
    w.q_base = p.cu_q[b];
    w.Lq = p.cu_q[b + 1] - w.q_base;
    w.k_base = p.cu_k[b];
    w.Lk = p.cu_k[b + 1] - w.k_base;
    w.qt = qt;
    // an item outside the sequence's tiles (a plan made for other lengths)
    // computes nothing
    w.valid = qt >= 0 && qt < (w.Lq + kBlockM - 1) / kBlockM;
    return w;
  }
  int lo = 0, hi = p.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.cu_q[mid] / kBlockM + mid <= t) lo = mid; else hi = mid - 1;
  }
  w.b = lo;
  w.q_base = p.cu_q[lo];
  w.Lq = p.cu_q[lo + 1] - w.q_base;
  w.k_base = p.cu_k[lo];
  w.Lk = p.cu_k[lo + 1] - w.k_base;
  const int lt = t - (w.q_base / kBlockM + lo);
  const int ntiles = (w.Lq + kBlockM - 1) / kBlockM;
  w.valid = lt < ntiles;
  w.qt = ntiles - 1 - lt;
  return w;
}

}  // namespace fa
