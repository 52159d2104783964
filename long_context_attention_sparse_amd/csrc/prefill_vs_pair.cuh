// Vertical-slash attention on pairs of neighbouring 64-row query blocks.
//
// Same operation as prefill_tile_kernel on vertical-slash patterns with 64-row query
// blocks ("Implementation: Sgl project Sglang Sparse Flash Attention", I/O Contract): row r
// of query block m attends to the union of block m's windows [w, w + block_N) and its
// columns, within [0, kv_len) and, when causal, up to its diagonal.
//
// Why pairs: a slash diagonal crosses query block m + 1 64 keys to the right of where it
// crosses block m, so the converter gives a run of adjacent windows of block m back in
// block m + 1 less its first window and plus one after its last.  Neighbouring blocks
// therefore name about half of their windows in common.  A workgroup of four waves takes
// both blocks of a pair (rows r0 .. r0 + 127; waves 0-1 block m, waves 2-3 block m + 1):
//   - shared steps: two windows named by both lists (128 keys, one K and one V tile of 128
//     rows) attended by all 128 rows, each loaded once for both blocks;
//   - split steps: one 64-key segment of block m's other windows or columns in tile rows
//     0..63, read by waves 0-1, beside one of block m + 1's in rows 64..127, read by waves
//     2-3.
// Each block attends each of its keys exactly once, so O and LSE are those of the one-block
// kernel up to the order of the float32 sums.  Which windows are common is found with a
// binary search of each staged list in the other; an entry past the staged prefix (more
// than kL windows) is simply taken as not shared, which only costs a second load.
//
// Per step the pipeline is the one of prefill_tile_kernel: [K_c in LDS] issue V_c -> S_c
// -> masks, row maximum -> wait, barrier -> issue K_{c+1} -> weights and P V_c -> wait,
// barrier.  LDS: 2 x 32 KB of tiles plus the staged lists (73 KB, two workgroups per CU).
#pragma once
#include <type_traits>

#include "tile.cuh"

namespace bsa {

// true when v is in the ascending LDS list p[0, n)
__device__ __forceinline__ bool lds_find_sorted(const int* p, int n, int v) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (lds_int(p, mid) < v) lo = mid + 1;
    else hi = mid;
  }
  return lo < n && lds_int(p, lo) == v;
}

// Number of lanes below this one whose bit is set in the wave-wide mask.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

template <int kRunPairs>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void vs_pair_kernel(PrefillArgs a) {
  constexpr int D = TD;
  constexpr int NT = 256;
  constexpr int CK = 128;  // tile rows: two 64-key segments
  constexpr int RS = D;
  constexpr int kL = NT;   // window entries of each block staged in LDS (one per thread)
  constexpr int kC = 768;  // column entries of each block staged in LDS
  __shared__ __attribute__((aligned(16))) uint16_t Kt[CK * RS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[CK * RS];
  __shared__ __attribute__((aligned(16))) int kid_s[CK];
  __shared__ int wl_s[2][kL];
  __shared__ int col_s[2][kC];
  __shared__ int scan_s[3][4];

  // (b, kv head, reversed pair, group member), every XCD on the same head as in the one-block
  // kernel, in runs of kRunPairs consecutive pairs dealt in mirrored rounds.  The last query
  // blocks of a head carry the most windows, so the XCDs must get even shares of a head:
  // plain rounds of 1, 2 or 4 pairs measured alike and 8 or 16 slower; mirrored rounds of 4 or
  // 8 pairs 4% faster than plain rounds of 4, of 16 or 32 slower again.  With the rotated
  // shared-step walk below, runs of 8 pairs beat runs of 4 by 2% (more neighbours per XCD
  // reading the same tiles), runs of 16 are 5% slower.
  const int npr = (a.nqb + 1) >> 1;
  const int item = head_sync_item_n<kRunPairs, true>(wg_x(), npr, a.n_items);
  const int g = item % a.G;
  int rest = item / a.G;
  const int prev = rest % npr;
  rest /= npr;
  const int hkv = rest % a.Hkv;
  const int b = rest / a.Hkv;
  const int h = hkv * a.G + g;
  const int m = 2 * (npr - 1 - prev);

  int q_start = 0, q_len = a.Sq, k_start = 0, kv_len = a.Sk;
  if (a.cu_q) {
    q_start = a.cu_q[b];
    q_len = a.cu_q[b + 1] - q_start;
    k_start = a.cu_k[b];
    kv_len = a.cu_k[b + 1] - k_start;
  }
  const int r0 = m * 64;
  if (r0 >= q_len) return;  // uniform: no barrier has run yet
  const bool has_b = m + 1 < a.nqb && r0 + 64 < q_len;
  const int delta = kv_len - q_len;

  const int t = tid_x();
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63;
  const int lq = l & 31, hh = l >> 5;
  const int hb = w >> 1;  // the wave's block: 0 = m, 1 = m + 1

  const uint16_t* qb = reinterpret_cast<const uint16_t*>(a.q.ptr) +
                       (a.cu_q ? (int64_t)q_start * a.q.ss : (int64_t)b * a.q.sb) + (int64_t)h * a.q.sh;
  const uint16_t* kbp = reinterpret_cast<const uint16_t*>(a.k.ptr) +
                        (a.cu_q ? (int64_t)k_start * a.k.ss : (int64_t)b * a.k.sb) + (int64_t)hkv * a.k.sh;
  const uint16_t* vbp = reinterpret_cast<const uint16_t*>(a.v.ptr) +
                        (a.cu_q ? (int64_t)k_start * a.v.ss : (int64_t)b * a.v.sb) + (int64_t)hkv * a.v.sh;

  const int row = r0 + w * 32 + lq;
  const bool row_ok = row < q_len;
  bf16x8 qreg[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const u32x4 v = row_ok ? ldg128(qb + (int64_t)row * a.q.ss + ks * 16 + hh * 8) : u32x4{0, 0, 0, 0};
    qreg[ks] = as_bf16x8(v);
  }

  // ---- the two blocks' lists ----
  const int ht = a.list_by_kv ? hkv : h;
  const int64_t lb0 = (int64_t)b * a.pat.s_b + (int64_t)ht * a.pat.s_h + (int64_t)m * a.pat.s_q;
  const int64_t lb1 = lb0 + a.pat.s_q;
  const bool keys = kv_len > 0;
  const int na = keys ? a.pat.count[lb0] : 0;
  const int nb = keys && has_b ? a.pat.count[lb1] : 0;
  const int nca = keys ? a.pat.col_count[lb0] : 0;
  const int ncb = keys && has_b ? a.pat.col_count[lb1] : 0;
  const int32_t* list_a = a.pat.index + lb0 * a.pat.cap;
  const int32_t* list_b = a.pat.index + lb1 * a.pat.cap;  // read only when has_b
  const int32_t* cols_a = a.pat.col_index + lb0 * a.pat.col_cap;
  const int32_t* cols_b = a.pat.col_index + lb1 * a.pat.col_cap;
  const int spe = a.pat.block_N / 64;  // 64-key segments per window

  const int sa = min(na, kL), sb = min(nb, kL);
  if (t < sa) wl_s[0][t] = list_a[t];
  if (t < sb) wl_s[1][t] = list_b[t];
  for (int x = t; x < min(nca, kC); x += NT) col_s[0][x] = cols_a[x];
  for (int x = t; x < min(ncb, kC); x += NT) col_s[1][x] = cols_b[x];
  __syncthreads();

  // Split each staged list into the windows both blocks name (kept in block m's order) and
  // the others; block m's list becomes [common | its own], block m + 1's [its own].
  const int va = t < sa ? wl_s[0][t] : 0;
  const int vb = t < sb ? wl_s[1][t] : 0;
  const bool fc = t < sa && lds_find_sorted(wl_s[1], sb, va);
  const bool fxa = t < sa && !fc;
  const bool fxb = t < sb && !lds_find_sorted(wl_s[0], sa, vb);
  const uint64_t bc = __ballot(fc), bxa = __ballot(fxa), bxb = __ballot(fxb);
  if (l == 0) {
    scan_s[0][w] = __popcll(bc);
    scan_s[1][w] = __popcll(bxa);
    scan_s[2][w] = __popcll(bxb);
  }
  __syncthreads();  // also: every read of the staged lists above is done
  int rc = lanes_below(bc), rxa = lanes_below(bxa), rxb = lanes_below(bxb);
  int nc = 0, nxa_s = 0, nxb_s = 0;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int c0 = scan_s[0][x], c1 = scan_s[1][x], c2 = scan_s[2][x];
    if (x < w) {
      rc += c0;
      rxa += c1;
      rxb += c2;
    }
    nc += c0;
    nxa_s += c1;
    nxb_s += c2;
  }
  nc = __builtin_amdgcn_readfirstlane(nc);
  nxa_s = __builtin_amdgcn_readfirstlane(nxa_s);
  nxb_s = __builtin_amdgcn_readfirstlane(nxb_s);
  if (fc) wl_s[0][rc] = va;
  if (fxa) wl_s[0][nc + rxa] = va;
  if (fxb) wl_s[1][rxb] = vb;
  __syncthreads();

  // windows of each block not shared: the staged ones, then every entry past the prefix
  const int nxa = nxa_s + max(0, na - kL), nxb = nxb_s + max(0, nb - kL);
  const int n_sh_seg = nc * spe;
  const int n_sh = (n_sh_seg + 1) >> 1;  // shared steps, two segments each
  const int nsa = nxa * spe + (nca + 63) / 64, nsb = nxb * spe + (ncb + 63) / 64;
  const int n_steps = n_sh + max(nsa, nsb);

  // this wave's block: columns and their count
  const int my_nc = hb ? ncb : nca;
  const int32_t* my_cols = hb ? cols_b : cols_a;
  const int* my_cols_s = col_s[hb];

  struct Seg {
    int key0 = 0, gbase = 0;
    bool valid = false, gathered = false, full = false;  // full: all 64 keys inside [0, kv_len)
  };
  auto window_seg = [&](int id, int part) -> Seg {
    Seg r;
    r.valid = true;
    r.key0 = id + part * 64;
    r.full = r.key0 >= 0 && r.key0 <= kv_len - 64;
    return r;
  };
  // Segment x (0 or 1) of shared step c (c < n_sh): common windows in block m's order, the
  // walk rotated by -(pair index) steps.  Near the diagonal the next pair's common windows are
  // this pair's shifted by 128 keys, one shared step; with the rotation neighbouring pairs
  // read the same tiles in the same step, while they are still in L2 (an XCD's 64 resident
  // pairs load about its whole L2 per step).
  const int rot = n_sh > 0 ? (n_sh - (m >> 1) % n_sh) % n_sh : 0;
  auto seg_shared = [&](int c, int x) -> Seg {
    c += rot;
    if (c >= n_sh) c -= n_sh;
    const int j = 2 * c + x;
    if (j >= n_sh_seg) return Seg{};
    const int e = spe == 2 ? j >> 1 : j;
    return window_seg(__builtin_amdgcn_readfirstlane(lds_int(wl_s[0], e)), j - e * spe);
  };
  // segment of block m + x (x = 0 or 1) in split step j (step n_sh + j)
  auto seg_split = [&](int j, int x) -> Seg {
    const int nx = x ? nxb : nxa, nxs = x ? nxb_s : nxa_s;
    if (j < nx * spe) {
      const int e = spe == 2 ? j >> 1 : j;
      int id;
      if (e < nxs) id = lds_int(x ? wl_s[1] : wl_s[0] + nc, e);
      else id = global_int(x ? list_b : list_a, kL + e - nxs);
      return window_seg(__builtin_amdgcn_readfirstlane(id), j - e * spe);
    }
    Seg r;
    const int ncol = x ? ncb : nca;
    if (j < nx * spe + (ncol + 63) / 64) {
      r.valid = true;
      r.gathered = true;
      r.gbase = (j - nx * spe) * 64;
    }
    return r;
  };
  // key of row i of a gathered segment of this wave's block, or -1 when absent
  auto col_key = [&](int i, const Seg& r) -> int {
    if (!r.valid) return -1;
    const int x = r.gbase + i;
    if (x >= my_nc) return -1;
    const int key = x < kC ? lds_int(my_cols_s, x) : global_int(my_cols, x);
    return (unsigned)key < (unsigned)kv_len ? key : -1;
  };

  // Direct loads: wave w fills tile rows 32w..32w+31 (segment w/2, segment rows
  // 32(w%2)..+31), as in prefill_tile_kernel.
  const int lrow = l >> 4, lslot = l & 15;
  const int srow0 = (w & 1) * 32;
  const uint32_t kx = (uint32_t)(lslot ^ lrow) << 4;
  const uint32_t vx = (uint32_t)(lslot ^ (lrow << 2)) << 4;
  const uint32_t k_lane = (uint32_t)(lrow * a.k.ss) * 2u, v_lane = (uint32_t)(lrow * a.v.ss) * 2u + vx;
  // contiguous segment (or an absent one: zeros) through a buffer resource sized to the rows
  // inside [0, kv_len)
  auto issue_win = [&](uint16_t* tile, const uint16_t* src, int64_t ss, bool is_k, const Seg& r)
                       __attribute__((always_inline)) {
    const int row0 = r.key0 + srow0;
    const int nrows = (r.valid && row0 >= 0) ? min(kv_len - row0, 32) : 0;
    const uint32_t row_bytes = (uint32_t)ss * 2u;
    const __amdgpu_buffer_rsrc_t rs =
        rows_rsrc(src + (int64_t)max(row0, 0) * ss, nrows > 0 ? (uint32_t)(nrows - 1) * row_bytes + 256u : 0u);
#pragma unroll
    for (int x = 0; x < 8; ++x)
      buffer_load_lds16(rs, tile + (w * 8 + x) * 4 * RS,
                        (uint32_t)(x * 4) * row_bytes + (is_k ? k_lane + (kx ^ ((x & 3) << 6)) : v_lane));
  };
  auto issue = [&](uint16_t* tile, const uint16_t* src, int64_t ss, bool is_k, const Seg& r)
                   __attribute__((always_inline)) {
    if (!r.gathered) {
      issue_win(tile, src, ss, is_k, r);
    } else {
      // the keys of this wave's 32 tile rows as record_kid stored them (absent ones as INT_MAX,
      // loaded as key 0 and masked): LDS reads only, so the loads below do not wait for a
      // column index read from global memory, whose wait would cover every load in flight
      int kk[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const int kid = kid_s[w * 32 + x * 4 + lrow];
        kk[x] = kid == 0x7fffffff ? 0 : kid;
      }
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const char* p = reinterpret_cast<const char*>(src + (int64_t)kk[x] * ss);
        __builtin_amdgcn_global_load_lds(p + (is_k ? (kx ^ ((x & 3) << 6)) : vx), BSA_LDS(tile + (w * 8 + x) * 4 * RS),
                                         16, 0, 0);
      }
    }
  };
  // a gathered segment records its key indices for the masks and the loads (tile rows of this
  // wave); every issue of a gathered segment follows the record of that segment
  auto record_kid = [&](const Seg& r) __attribute__((always_inline)) {
    if (r.gathered && l < 32) {
      const int key = col_key(srow0 + l, r);
      kid_s[w * 32 + l] = key >= 0 ? key : 0x7fffffff;
    }
  };

  // per-lane LDS offsets of the MFMA operands: K rows of step ks at koff0 ^ 16 ks (the
  // swizzle only flips the piece bits), V^T pieces of dim block db at voff0 ^ 32 db
  const int koff0 = lq * RS + ((hh ^ k_swz(lq)) << 3);
  const int tg = l >> 4, tr = l & 15;
  const int vrow = (tg >> 1) * 4 + (tr >> 2);
  const int vcol0 = (tg & 1) * 16 + (tr & 3) * 4;
  const int voff0 = vrow * RS + (((vcol0 >> 3) ^ v_swz(vrow)) << 3) + (vcol0 & 7);
  auto koff = [&](int ks) { return koff0 ^ (ks << 4); };
  auto voff = [&](int db) { return voff0 ^ (db << 5); };

  float m_run = kNegInf, l_run = 0.f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int x = 0; x < D / 32; ++x) oacc[x] = f32x16{};

  // -inf for absent keys and, when causal, keys after the row's diagonal (tile block kb of
  // 32 keys lies in segment kb / 2)
  const int wrow_min = r0 + w * 32;
  // Shared steps hold windows only.  Split steps also hold gathered columns; their mask takes
  // one path for both kinds, the key of each element being the recorded column index or the
  // window's key (two alternative paths would make the compiler copy the scores around them).
  auto mask_block = [&](f32x16& s, int kb, const Seg& r, auto cols_c) __attribute__((always_inline)) {
    constexpr bool COLS = decltype(cols_c)::value;
    const int lim = a.causal ? row + delta : 0x7ffffffe;
    const int half = (kb & 1) * 32;
    const bool need = (COLS && r.gathered) || !r.full || (a.causal && r.key0 + half + 31 > wrow_min + delta);
    if (!need) return;
    if constexpr (COLS) {
      // present gathered keys lie in [0, kv_len), absent ones are recorded as INT_MAX
      const int lim_eff = r.gathered ? lim : (r.valid ? min(lim, kv_len - 1) : -1);
      const int base = r.key0 + half;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int4 k4 = *reinterpret_cast<const int4*>(kid_s + kb * 32 + q4 * 8 + hh * 4);
        const int kk[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = r.gathered ? kk[e] : base + q4 * 8 + hh * 4 + e;
          if (key > lim_eff || key < 0) s[q4 * 4 + e] = kNegInf;
        }
      }
    } else {
      const int hi = r.valid ? min(lim, kv_len - 1) - r.key0 - half : -1;
      const int lo = -r.key0 - half;
#pragma unroll
      for (int rg = 0; rg < 16; ++rg) {
        const int kl = (rg >> 2) * 8 + hh * 4 + (rg & 3);
        if (kl > hi || kl < lo) s[rg] = kNegInf;
      }
    }
  };

  // S over NBW 32-key tile blocks from tile block kb0, masks and the row maximum
  auto s_phase = [&](auto nbw_c, int kb0, f32x16* s, const Seg& seg0, const Seg& seg1) __attribute__((always_inline)) {
    constexpr int NBW = decltype(nbw_c)::value;
#pragma unroll
    for (int kb = 0; kb < NBW; ++kb) s[kb] = f32x16{};
    const uint16_t* kt = Kt + kb0 * 32 * RS;
    u32x4 av[2][NBW];
#pragma unroll
    for (int kb = 0; kb < NBW; ++kb) av[0][kb] = *reinterpret_cast<const u32x4*>(kt + kb * 32 * RS + koff(0));
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      if (ks + 1 < D / 16) {
#pragma unroll
        for (int kb = 0; kb < NBW; ++kb)
          av[(ks + 1) & 1][kb] = *reinterpret_cast<const u32x4*>(kt + kb * 32 * RS + koff(ks + 1));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kb = 0; kb < NBW; ++kb) s[kb] = mfma32x32x16(as_bf16x8(av[ks & 1][kb]), qreg[ks], s[kb]);
      __builtin_amdgcn_sched_barrier(0);
    }
    softcap_n<NBW>(s, a.cap_in, a.cap_out);
#pragma unroll
    for (int kb = 0; kb < NBW; ++kb) {
      if (NBW == 4) mask_block(s[kb], kb, kb < 2 ? seg0 : seg1, std::false_type{});
      else mask_block(s[kb], kb0 + kb, seg0, std::true_type{});  // split step: seg0 is this wave's segment
    }
    softmax_max_n<NBW>(s, a.scale_log2, m_run, l_run, oacc);
  };
  // weights and P V over the same tile blocks
  auto pv_phase = [&](auto nbw_c, int kb0, f32x16* s) __attribute__((always_inline)) {
    constexpr int NBW = decltype(nbw_c)::value;
    const uint16_t* vt = Vt + kb0 * 32 * RS;
    u32x4 vpre[2][D / 32];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const u32x2 lo = ds_read_tr16(vt + ks * 16 * RS + voff(db));
        const u32x2 hi = ds_read_tr16(vt + (ks * 16 + 8) * RS + voff(db));
        vpre[ks][db] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
    const float m_use = m_run == kNegInf ? 0.f : m_run;
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < NBW; ++kb) {
      uint32_t pk[8];
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        const float p0 = exp2_fast(fmaf(s[kb][r], a.scale_log2, -m_use));
        const float p1 = exp2_fast(fmaf(s[kb][r + 1], a.scale_log2, -m_use));
        const float p2 = exp2_fast(fmaf(s[kb][r + 2], a.scale_log2, -m_use));
        const float p3 = exp2_fast(fmaf(s[kb][r + 3], a.scale_log2, -m_use));
        pk[r / 2] = pack_bf16x2(p0, p1);
        pk[r / 2 + 1] = pack_bf16x2(p2, p3);
        psum += (p0 + p1) + (p2 + p3);
      }
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int ks = kb * 2 + x;
        const u32x4 pb = {pk[x * 4], pk[x * 4 + 1], pk[x * 4 + 2], pk[x * 4 + 3]};
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          u32x4 av;
          if (ks < 2) {
            av = vpre[ks < 2 ? ks : 0][db];
          } else {
            const u32x2 lo = ds_read_tr16(vt + ks * 16 * RS + voff(db));
            const u32x2 hi = ds_read_tr16(vt + (ks * 16 + 8) * RS + voff(db));
            av = u32x4{lo[0], lo[1], hi[0], hi[1]};
          }
          oacc[db] = mfma32x32x16(as_bf16x8(av), as_bf16x8(pb), oacc[db]);
        }
      }
    }
    l_run += psum;
  };

  // ---- step loop ----
  // a split step only needs this wave's block's segment: both copies hold it
  Seg cur0, cur1;
  if (n_sh > 0) {
    cur0 = seg_shared(0, 0);
    cur1 = seg_shared(0, 1);
  } else {
    cur0 = cur1 = seg_split(0, hb);
  }
  if (n_steps > 0) {
    const Seg mine = hb ? cur1 : cur0;
    record_kid(mine);
    issue(Kt, kbp, a.k.ss, true, mine);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // one step: shared (NBW = 4 tile blocks for every wave) or split (NBW = 2, this wave's
  // block's segment).  NEXT_SHARED: the next step is a shared one too, so neither this step's
  // nor the next one's segments are gathered columns (the loop over those steps carries no
  // gathered-load code).
  auto step = [&](auto nbw_c, auto next_shared_c, int c) __attribute__((always_inline)) {
    constexpr int NBW = decltype(nbw_c)::value;
    constexpr bool NEXT_SHARED = decltype(next_shared_c)::value;
    const bool more = NEXT_SHARED || c + 1 < n_steps;
    const Seg mine = hb ? cur1 : cur0;
    // (a split step whose segment of this wave's block is absent runs on zeros, all masked:
    // it adds nothing to the rows, and a test around the products would cost more)
    if (NBW == 4) issue_win(Vt, vbp, a.v.ss, false, mine);
    else issue(Vt, vbp, a.v.ss, false, mine);
    f32x16 s[NBW];
    if (NBW == 4) s_phase(nbw_c, 0, s, cur0, cur1);
    else s_phase(nbw_c, 2 * hb, s, mine, mine);
    // V_c is in LDS from every wave, and every wave is done reading K_c and the indices
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    Seg nxt0, nxt1;
    if (NEXT_SHARED) {
      nxt0 = seg_shared(c + 1, 0);
      nxt1 = seg_shared(c + 1, 1);
      issue_win(Kt, kbp, a.k.ss, true, hb ? nxt1 : nxt0);
    } else if (more) {
      // the next step is a split one (this is the last shared step or a split step).  Its
      // key indices are recorded before its loads are issued: a column index past the staged
      // ones is read from global memory, and the wait for that read would also wait for every
      // load issued before it.
      nxt0 = nxt1 = seg_split(c + 1 - n_sh, hb);
      record_kid(nxt0);
      issue(Kt, kbp, a.k.ss, true, nxt0);
    }
    pv_phase(nbw_c, NBW == 4 ? 0 : 2 * hb, s);
    if (more) {
      // K_{c+1} is in LDS and every wave is done reading V_c
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      cur0 = nxt0;
      cur1 = nxt1;
    }
  };
  using shared_c = std::integral_constant<int, 4>;
  using split_c = std::integral_constant<int, 2>;
  int c = 0;
  for (; c + 1 < n_sh; ++c) step(shared_c{}, std::true_type{}, c);
  if (c < n_sh) step(shared_c{}, std::false_type{}, c++);  // the last shared step
  for (; c < n_steps; ++c) step(split_c{}, std::false_type{}, c);

  if (row_ok) {
    const int64_t ob = (a.cu_q ? (int64_t)(q_start + row) * a.o.ss : (int64_t)b * a.o.sb + (int64_t)row * a.o.ss) +
                       (int64_t)h * a.o.sh;
    float* lp = nullptr;
    if (a.lse) lp = a.lse + (a.cu_q ? (int64_t)h * a.cu_q[a.B] + q_start + row : ((int64_t)b * a.Hq + h) * a.Sq + row);
    write_row(a.o, ob, lp, oacc, m_run, l_run, hh);
  }
}

}  // namespace bsa
