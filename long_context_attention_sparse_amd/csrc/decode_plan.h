// Decode launch planning: when the decode kernel takes a problem, how the G query heads of a
// kv head are packed, and how the key range of each segment is split over workgroups.
#pragma once
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>

#include "args.cuh"
#include "bsa.h"
#include "host_args.h"
#include "launch.h"

namespace bsa {

struct SegPlan {
  int n_entries = 0, cpe = 1, eps = 1, splits = 0;
};

struct DecodePlan {
  bool use = false;
  int Gp = 1, R = 0;
};

// Packing rule: the G query heads of a kv head share one workgroup when they share
// its key set; with the query positions they must fit one 16-column MFMA tile.
inline DecodePlan plan_decode(const bsa_problem& p, const bsa_pattern* pat) {
  DecodePlan d;
  const int kind = pat ? pat->kind : BSA_PAT_DENSE;
  if (p.cu_seqlens_q || kind == BSA_PAT_VS) return d;
  const int G = p.Hq / p.Hkv;
  const bool shared = kind == BSA_PAT_DENSE || pat->Ht == p.Hkv;
  d.Gp = shared ? G : 1;
  d.R = d.Gp * p.Sq;
  if (d.R > 16) return d;
  if (kind == BSA_PAT_BLOCK && p.Sq > pat->block_M) return d;
  d.use = true;
  return d;
}

inline SegPlan seg_entries(int Sk, const bsa_pattern* pat) {
  SegPlan s;
  if (!pat || pat->kind == BSA_PAT_DENSE) {
    s.n_entries = (Sk + 63) / 64;
    s.cpe = 1;
  } else {
    s.n_entries = pat->cap;
    s.cpe = pat->block_N / 64;
  }
  return s;
}

// Compute units of the current device (cached per device).
inline int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

#ifndef BSA_DECODE_ROUNDS
#define BSA_DECODE_ROUNDS 4
#endif
constexpr int kDecodeWgPerCu = 4;                  // resident decode workgroups per CU (128 VGPRs, 36 KB LDS)
constexpr int kDecodeRounds = BSA_DECODE_ROUNDS;   // whole rounds of resident workgroups per launch
constexpr int kMaxChunksPerSplit = 96;             // more rounds when splits would get longer than this

// Split the segments of one decode launch: the splits of a group are a whole number of
// rounds of resident workgroups (no quarter-full last round), shared between segments in
// proportion to their chunk counts, so every workgroup streams a similar number of chunks.
inline void split_segments(SegPlan* segs, int nseg, int groups) {
  long total = 0;
  for (int i = 0; i < nseg; ++i) total += (long)std::max(0, segs[i].n_entries) * segs[i].cpe;
  const long capacity = (long)device_cus() * kDecodeWgPerCu;
  long rounds = kDecodeRounds;
  while (total * groups > rounds * capacity * kMaxChunksPerSplit) ++rounds;
  long per_group = std::max<long>(1, (rounds * capacity + groups / 2) / groups);
  per_group = std::max<long>(per_group, nseg);
  long assigned = 0;
  for (int i = 0; i < nseg; ++i) {
    SegPlan& s = segs[i];
    if (s.n_entries <= 0) {
      s.eps = 1;
      s.splits = 1;
      ++assigned;
      continue;
    }
    const long chunks = (long)s.n_entries * s.cpe;
    long want = i == nseg - 1 ? per_group - assigned : (per_group * chunks + total / 2) / std::max<long>(total, 1);
    want = std::max<long>(1, std::min<long>(want, s.n_entries));
    s.eps = (int)((s.n_entries + want - 1) / want);
    s.splits = (s.n_entries + s.eps - 1) / s.eps;
    assigned += s.splits;
  }
}

inline size_t partial_bytes(const bsa_problem& p, int slots) {
  const size_t rows = (size_t)p.B * p.Sq * p.Hq;
  return (size_t)slots * rows * (p.D + 1) * sizeof(float) + 256;
}

inline DecodeSeg make_seg(const bsa_tensor& k, const bsa_tensor& v, const bsa_pattern* pat, int Sk, int causal,
                   const SegPlan& sp, int slot0) {
  DecodeSeg s{};
  s.k = targ(k);
  s.v = targ(v);
  s.pat = parg(pat);
  s.Sk = Sk;
  s.causal = causal != 0;
  s.n_entries = sp.n_entries;
  s.cpe = sp.cpe;
  s.eps = sp.eps;
  s.splits = sp.splits;
  s.slot0 = slot0;
  return s;
}

// One decode launch over one or two segments; writes (O, LSE) directly when o is given
// (single segment, single split), partial slots otherwise.
inline bsa_status run_decode(const bsa_problem& p, const DecodePlan& d, const bsa_tensor& q, const DecodeSeg* segs, int nseg,
                      float* part_o, float* part_lse, const bsa_tensor* o, float* lse, hipStream_t st) {
  DecodeArgs a{};
  a.q = targ(q);
  a.nseg = nseg;
  a.seg[0] = segs[0];
  if (nseg > 1) a.seg[1] = segs[1];
  a.B = p.B;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.Sq = p.Sq;
  a.G = p.Hq / p.Hkv;
  a.Gp = d.Gp;
  a.R = d.R;
  a.scale_log2 = scale_of(p) * kLog2e;
  cap_consts(p, a.cap_in, a.cap_out);
  if (o) {
    a.direct = 1;
    a.o = oarg(*o);
    a.lse = lse;
  } else {
    a.direct = 0;
    a.part_o = part_o;
    a.part_lse = part_lse;
  }
  int gx = 0;
  for (int i = 0; i < nseg; ++i) gx += segs[i].splits;
  launch_decode(a, p.D, gx, p.Hq / d.Gp, p.B, st);
  return launch_status();
}

// Split plan of bsa_fwd on the decode path (one segment).
inline SegPlan fwd_decode_plan(const bsa_problem& p, const bsa_pattern* pat, const DecodePlan& d) {
  SegPlan sp = seg_entries(p.Sk, pat);
  split_segments(&sp, 1, p.B * (p.Hq / d.Gp));
  return sp;
}

// Partial slots of the fused speculative + repair launch (decode shapes), or 2.
inline void speculative_plan(const bsa_problem& p, int Sk_spec, const bsa_pattern* missed, SegPlan segs[2],
                             DecodePlan* dp) {
  *dp = plan_decode(p, missed);
  segs[0] = seg_entries(Sk_spec, nullptr);
  segs[1] = seg_entries(p.Sk, missed);
  if (dp->use) {
    split_segments(segs, 2, p.B * (p.Hq / dp->Gp));
  } else {
    for (int i = 0; i < 2; ++i) {
      segs[i].eps = std::max(1, segs[i].n_entries);
      segs[i].splits = 1;
    }
  }
}

}  // namespace bsa
