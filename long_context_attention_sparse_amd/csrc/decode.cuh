// Split-KV decode kernel: few query rows per key/value head, many keys.
//
// Computes attention restricted to listed key blocks ("Sparse FlashAttention
// with Incremental Repair", Usage 1) for problems whose query rows per
// key/value head fit one 16-wide MFMA tile: the G query heads that share a
// key/value head (and share its block list) are packed together with the Sq
// query positions into at most 16 rows, so every K/V byte is read once per
// group.  A launch holds one or two segments — key sets over possibly
// different K/V tensors, e.g. the speculative pass and the repair pass of
// Usage 2 — and each segment's list is cut into splits.  Each workgroup
// streams its split's 64-key chunks through LDS and writes either the final
// (O, LSE) or a float32 partial that the combine kernel merges (log-sum-exp
// combine, same page, What's in this fork).
//
// Work decomposition: grid (splits of all segments, head groups, B), 256
// threads = 4 waves.  The split's block ids are staged in LDS first, so the
// address of every chunk is known without a dependent global load.  Per
// 64-key chunk every thread loads D/32 16-byte pieces of K and of V
// (coalesced: K 16 or 8 lanes per 256/128-byte key row, V at head dim 128
// 8 lanes per 128-byte half row), both with the streaming cache policy; K
// goes to LDS row-major, V is transposed in registers and stored
// key-contiguous per head-dim row.  Wave w owns keys 16w..16w+15 of the chunk and keeps its own
// running (max, sum, O^T); the four waves merge once at the end.
//   S^T = K Q^T    : v_mfma_f32_16x16x32_bf16, D/32 per chunk (lane = query col)
//   O^T += V^T P^T : v_mfma_f32_16x16x16_bf16, D/16 per chunk
// The next chunk's loads are issued before the current chunk's MFMAs.
#pragma once
#include "common.cuh"

namespace bsa {




template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void decode_kernel(DecodeArgs a) {
  constexpr int PIECES = D / 8;                // 16-byte pieces per key row
  constexpr int KEYS_PER_PASS = 256 / PIECES;  // key rows one pass of 256 threads covers
  constexpr int L = 64 / KEYS_PER_PASS;        // consecutive keys per thread (4 or 2)
  constexpr int KS = D + 8;                    // Ks row stride in bf16 (pad: conflict-free b128 reads)
  constexpr int VSTR = D == 128 ? 64 + 4 : 64 + 8;  // Vt row stride in bf16 (conflict-free stores and reads)
  constexpr int LDS_KV = (64 * KS + D * VSTR) * 2;
  constexpr int MS = D + 4;                    // merge row stride in floats (conflict-free b128 stores)
  constexpr int LDS_MERGE = (4 * 16 * MS + 3 * 64) * 4;
  constexpr int LDS_BYTES = LDS_KV > LDS_MERGE ? LDS_KV : LDS_MERGE;
  __shared__ __attribute__((aligned(16))) unsigned char smem[LDS_BYTES];
  __shared__ int ents[kDecodeEntsLds];
  uint16_t* Ks = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Vt = Ks + 64 * KS;

  const int t = threadIdx.x;
  const int w = t >> 6, l = t & 63;
  const int lr = l & 15, kg = l >> 4;
  const int hg = blockIdx.y, b = blockIdx.z;
  const int si = (a.nseg > 1 && (int)blockIdx.x >= a.seg[0].splits) ? 1 : 0;
  const DecodeSeg& sg = a.seg[si];
  const int sp = blockIdx.x - (si ? a.seg[0].splits : 0);

  // ---- query rows of this lane (MFMA column lr) ----
  const int rho = lr;
  const bool row_ok = rho < a.R;
  const int s_row = row_ok ? rho / a.Gp : 0;
  const int hq_row = hg * a.Gp + (row_ok ? rho % a.Gp : 0);
  const int hkv = (hg * a.Gp) / a.G;
  const int lim = sg.causal ? s_row + (sg.Sk - a.Sq) : 0x7fffffff;

  bf16x8 qreg[D / 32];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q.ptr) + b * a.q.sb + (int64_t)s_row * a.q.ss +
                         (int64_t)hq_row * a.q.sh + kg * 8;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      u32x4 v = row_ok ? ldg128(qp + ks * 32) : u32x4{0, 0, 0, 0};
      qreg[ks] = as_bf16x8(v);
    }
  }

  // ---- this split's entries, staged in LDS ----
  int n_list;
  const int32_t* list = nullptr;
  if (sg.pat.kind == 0) {
    n_list = sg.n_entries;
  } else {
    const int64_t lb = b * sg.pat.s_b + hg * sg.pat.s_h;
    n_list = sg.pat.count[lb];
    list = sg.pat.index + lb * sg.pat.cap;
  }
  const int e0 = sp * sg.eps;
  const int e1 = min(n_list, e0 + sg.eps);
  const int cpe = sg.cpe;
  const int nchunks = e1 > e0 ? (e1 - e0) * cpe : 0;
  if (list && t < kDecodeEntsLds && e0 + t < e1) ents[t] = list[e0 + t];

  const int c = t % PIECES, kk = t / PIECES;
  const uint16_t* kbase = reinterpret_cast<const uint16_t*>(sg.k.ptr) + b * sg.k.sb + (int64_t)hkv * sg.k.sh + c * 8;
  const uint16_t* vbase = reinterpret_cast<const uint16_t*>(sg.v.ptr) + b * sg.v.sb + (int64_t)hkv * sg.v.sh + c * 8;
  const int Sk = sg.Sk;

  auto chunk_key0 = [&](int ci) -> int {
    const int el = ci / cpe;
    if (!list) return (e0 + el) * 64;
    const int id = el < kDecodeEntsLds ? ents[el] : list[e0 + el];
    return id * (64 * cpe) + (ci - el * cpe) * 64;
  };

  // V for head dim 128: each thread owns 4 consecutive keys (4-key group kv) of one 16-byte
  // head-dim piece (cv) and stores them transposed.  Wave w takes the pieces of one 128-byte
  // half of each key row (8(w & 1) .. + 7) for the key groups of one half of the chunk
  // (8(w >> 1) .. + 7), lane l group l % 8 and piece l / 8: every load instruction reads whole
  // 128-byte lines, and with the 68-element V^T row stride the stores of each 32 lanes and the
  // P V reads hit distinct banks.  Head dim 64 uses the K mapping.
  constexpr bool kVGroups = D == 128;
  const int kv = 8 * (w >> 1) + (l & 7), cv = 8 * (w & 1) + (l >> 3);
  const uint16_t* vbase2 = reinterpret_cast<const uint16_t*>(sg.v.ptr) + b * sg.v.sb + (int64_t)hkv * sg.v.sh + cv * 8;
  // K and V are read once per launch, each 128-byte line by one load instruction, so both go
  // through nontemporal loads (the streaming cache policy), which keep them from displacing
  // other lines: K that way made the speculative + sparse launch 8% faster, V another 2% once
  // its mapping covered whole lines.  (With V lanes over half lines, the other half read by
  // the next wave, nontemporal V loads fetched 4% of the bytes twice and ran 3% slower.)
  auto ldg128_nt = [](const uint16_t* p) __attribute__((always_inline)) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  };
  u32x4 kr[L], vr[L];
  auto load_chunk = [&](int key0) {
#pragma unroll
    for (int j = 0; j < L; ++j) {
      const int key = key0 + kk * L + j;
      const bool ok = (unsigned)key < (unsigned)Sk;
      kr[j] = ok ? ldg128_nt(kbase + (int64_t)key * sg.k.ss) : u32x4{0, 0, 0, 0};
      if constexpr (kVGroups) {
        const int vkey = key0 + kv * 4 + j;
        vr[j] = (unsigned)vkey < (unsigned)Sk ? ldg128_nt(vbase2 + (int64_t)vkey * sg.v.ss) : u32x4{0, 0, 0, 0};
      } else {
        vr[j] = ok ? ldg128(vbase + (int64_t)key * sg.v.ss) : u32x4{0, 0, 0, 0};
      }
    }
  };

  float m_run = kNegInf, l_run = 0.f, le_run = 0.f;
  f32x4 oacc[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // the first chunk's address comes straight from global memory, so its loads are in
  // flight while the block ids are being staged
  int key0_next = nchunks > 0 ? (list ? list[e0] * (64 * cpe) : e0 * 64) : 0;
  if (nchunks > 0) load_chunk(key0_next);
  __syncthreads();

  for (int ci = 0; ci < nchunks; ++ci) {
    const int key0 = key0_next;
    __syncthreads();
    // K row-major; V transposed to [d][key]
#pragma unroll
    for (int j = 0; j < L; ++j) *reinterpret_cast<u32x4*>(Ks + (kk * L + j) * KS + c * 8) = kr[j];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint16_t* dst0 = kVGroups ? Vt + (cv * 8 + 2 * p) * VSTR + kv * 4 : Vt + (c * 8 + 2 * p) * VSTR + kk * L;
      uint16_t* dst1 = dst0 + VSTR;
      if constexpr (L == 4) {
        u32x2 ev = {lo_halves(vr[0][p], vr[1][p]), lo_halves(vr[2][p], vr[3][p])};
        u32x2 od = {hi_halves(vr[0][p], vr[1][p]), hi_halves(vr[2][p], vr[3][p])};
        *reinterpret_cast<u32x2*>(dst0) = ev;
        *reinterpret_cast<u32x2*>(dst1) = od;
      } else {
        *reinterpret_cast<uint32_t*>(dst0) = lo_halves(vr[0][p], vr[1][p]);
        *reinterpret_cast<uint32_t*>(dst1) = hi_halves(vr[0][p], vr[1][p]);
      }
    }
    __syncthreads();
    if (ci + 1 < nchunks) {
      key0_next = chunk_key0(ci + 1);
      load_chunk(key0_next);
    }

    // S^T for this wave's 16 keys
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const u32x4 kv = *reinterpret_cast<const u32x4*>(Ks + (w * 16 + lr) * KS + ks * 32 + kg * 8);
      s = mfma16x16x32(as_bf16x8(kv), qreg[ks], s);
    }
    if (a.cap_in != 0.f) {
#pragma unroll
      for (int r = 0; r < 4; ++r) s[r] = softcap_score(s[r], a.cap_in, a.cap_out);
    }
    float sc[4];
    float cmax = kNegInf;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = key0 + w * 16 + kg * 4 + r;
      const bool ok = (unsigned)key < (unsigned)Sk && key <= lim;
      sc[r] = ok ? s[r] * a.scale_log2 : kNegInf;
      cmax = fmaxf(cmax, sc[r]);
    }
    cmax = fmaxf(cmax, shfl_xor_f(cmax, 16));
    cmax = fmaxf(cmax, shfl_xor_f(cmax, 32));
    const float m_new = fmaxf(m_run, cmax);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2_fast(m_run - m_use);
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = exp2_fast(sc[r] - m_use);
    const u32x2 pb = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
    // O is normalised by the rounded weights the PV product uses (an exact convex
    // combination of V rows, so a dominant key's rounding cancels)
    l_run = bf16x2_sum_acc(pb[1], bf16x2_sum_acc(pb[0], l_run * alpha));
    // exact normaliser for LSE
    le_run = le_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      oacc[db] *= alpha;
      const u32x2 vv = *reinterpret_cast<const u32x2*>(Vt + (db * 16 + lr) * VSTR + w * 16 + kg * 4);
      oacc[db] = mfma16x16x16(as_bf16x4(vv), as_bf16x4(pb), oacc[db]);
    }
  }

  // ---- merge the four waves ----
  l_run += shfl_xor_f(l_run, 16);
  l_run += shfl_xor_f(l_run, 32);
  le_run += shfl_xor_f(le_run, 16);
  le_run += shfl_xor_f(le_run, 32);
  __syncthreads();
  float* mo = reinterpret_cast<float*>(smem);  // [4][16][MS]
  float* mm = mo + 4 * 16 * MS;                // [4][16]
  float* ml = mm + 64;
  float* mle = ml + 64;
#pragma unroll
  for (int db = 0; db < D / 16; ++db) *reinterpret_cast<f32x4*>(mo + (w * 16 + lr) * MS + db * 16 + kg * 4) = oacc[db];
  if (kg == 0) {
    mm[w * 16 + lr] = m_run;
    ml[w * 16 + lr] = l_run;
    mle[w * 16 + lr] = le_run;
  }
  __syncthreads();

  constexpr int DPT = D / 16;  // head-dim values per thread in the merge (4 per 64-wide half)
  const int row = t >> 4, dp = t & 15;
  if (row >= a.R) return;
  float M = kNegInf;
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, mm[ww * 16 + row]);
  float wt[4], Lt = 0.f, Le = 0.f;
  const float Mu = M == kNegInf ? 0.f : M;
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) {
    wt[ww] = exp2_fast(mm[ww * 16 + row] - Mu);
    Lt += wt[ww] * ml[ww * 16 + row];
    Le += wt[ww] * mle[ww * 16 + row];
  }
  const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
  const float lse_val = Le > 0.f ? (M + log2f(Le)) * kLn2 : kNegInf;
  // this thread's head-dim values: 4 consecutive ones in each 64-wide half (d = 64j + 4dp + e),
  // so that the 16 threads of a row read one contiguous 256-byte stretch per instruction
  float out[DPT];
#pragma unroll
  for (int j = 0; j < D / 64; ++j) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) acc += wt[ww] * *reinterpret_cast<const f32x4*>(mo + (ww * 16 + row) * MS + j * 64 + dp * 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) out[j * 4 + e] = acc[e] * inv;
  }
  const int s_o = row / a.Gp;
  const int hq_o = hg * a.Gp + row % a.Gp;
  if (a.direct) {
    const int64_t off = b * a.o.sb + (int64_t)s_o * a.o.ss + (int64_t)hq_o * a.o.sh + dp * 4;
#pragma unroll
    for (int j = 0; j < D / 64; ++j) store4(a.o, off + j * 64, out[j * 4], out[j * 4 + 1], out[j * 4 + 2], out[j * 4 + 3]);
    if (dp == 0 && a.lse) a.lse[((int64_t)b * a.Hq + hq_o) * a.Sq + s_o] = lse_val;
  } else {
    const int64_t slot = sg.slot0 + sp;
    float* po = a.part_o + (((slot * a.B + b) * a.Sq + s_o) * a.Hq + hq_o) * D + dp * 4;
#pragma unroll
    for (int j = 0; j < D / 64; ++j)
      *reinterpret_cast<f32x4*>(po + j * 64) = f32x4{out[j * 4], out[j * 4 + 1], out[j * 4 + 2], out[j * 4 + 3]};
    if (dp == 0) a.part_lse[((slot * a.B + b) * a.Hq + hq_o) * a.Sq + s_o] = lse_val;
  }
}

}  // namespace bsa
