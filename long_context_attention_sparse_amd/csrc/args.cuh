// Plain argument blocks of the kernels, filled on the host by the C ABI layer and
// passed by value to the launches (launch.h).
#pragma once
#include <stdint.h>

namespace bsa {

struct TensorArg {
  const void* ptr;
  int64_t sb, ss, sh;  // element strides (batch, token, head); head dim contiguous
};

struct OutArg {
  void* ptr;
  int64_t sb, ss, sh;
  int f32;  // 1: float32 output, 0: bf16
};

struct PatternArg {
  int kind;  // 0 dense, 1 block lists, 2 vertical-slash
  int block_M, block_N, cap, col_cap;
  const int32_t* count;
  const int32_t* index;
  const int32_t* col_count;
  const int32_t* col_index;
  int64_t s_b, s_h, s_q;
};

constexpr int kDecodeEntsLds = 256;    // block ids of a decode split staged in LDS (later ones read from global)
constexpr int kVSConvThreads = 64;     // conversion workgroup size (one query block per thread)
constexpr int kVSConvLdsInts = 16384;  // slash entries staged in LDS for the window walk (longer lists stay in global)
constexpr int kVSColLdsInts = 4096;    // windows of a query block staged in LDS for the column test
constexpr int kThreshMaxCand = 4096;   // threshold selection: query blocks per row (LDS candidates)
constexpr int kSelTile = 1024;         // selected attention: token positions per index workgroup
constexpr int kSelMaxBlocks = 8192;    // selected attention: key blocks per sequence (LDS histogram)
constexpr int kBwdChunk = 128;         // backward: 32-row query slabs per dK/dV workgroup
constexpr int kBwdListLds = 256;       // backward dQ: pattern-list entries of a query block staged in LDS

struct DecodeSeg {
  TensorArg k, v;
  PatternArg pat;       // kind 0: dense over [0, Sk)
  int Sk, causal;
  int n_entries;        // dense: number of 64-key chunks; lists: entries per list (cap)
  int cpe;              // 64-key chunks per entry
  int eps;              // entries per split
  int splits;           // splits of this segment (grid x range)
  int slot0;            // first partial slot written by this segment
};

struct DecodeArgs {
  TensorArg q;
  OutArg o;        // final output (direct mode)
  float* lse;      // final LSE [B, Hq, Sq] or nullptr (direct mode)
  float* part_o;   // partials [slots, B, Sq, Hq, D] (split mode)
  float* part_lse; // partials [slots, B, Hq, Sq] (split mode)
  DecodeSeg seg[2];
  int nseg;
  int B, Hq, Hkv, Sq, G, Gp, R;
  int direct;
  float scale_log2;  // softmax_scale * log2(e)
  float cap_in, cap_out;  // softcap constants (softcap_score); cap_in == 0: no softcap
};

struct PrefillArgs {
  TensorArg q, k, v;
  OutArg o;
  float* lse;
  PatternArg pat;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int B, Hq, Hkv, G, Sq, Sk;  // Sq/Sk: lengths (varlen: maxima)
  int nqb;                    // query blocks per (b, h) in the grid
  int list_by_kv;             // lists indexed by kv head (1) or query head (0)
  int causal;
  float scale_log2;
  float cap_in, cap_out;      // softcap constants (softcap_score); cap_in == 0: no softcap
  int n_items;
  int partial;                // 1: partials of epp entries each into part_o / part_lse
  int epp, n_part;
  float* part_o;              // [n_part, B, Sq, Hq, D]
  float* part_lse;            // [n_part, B, Hq, Sq]
};

struct GatedArgs {
  TensorArg q, k, v;
  OutArg o;
  float* lse;
  const float* T;      // [B, Hq, nqb]
  uint8_t* keep;       // [B, Hq, nqb, nqb] or nullptr
  float* tmax;         // [B, Hq, nqb, nqb] or nullptr
  int B, Hq, Hkv, G, S, nqb;
  float scale, scale_log2;
  int n_items;
  int count_skipped;   // 1: a skipped tile's scores stay in the running maximum and normalisers
};

// Selected attention (top-k key blocks per query token, key-block-outer).  Tokens are
// numbered t = b * Sq + position (fixed length) or by their packed index (varlen); a
// selection entry is sel[(t * Hkv + hkv) * topk + slot], a key block of the token's own
// sequence or -1.
struct SelArgs {
  TensorArg q, k, v;
  const int32_t* sel;
  const int32_t* cu_q;   // varlen prefix sums or null
  const int32_t* cu_k;
  int B, Hq, Hkv, G, Sq, Sk;  // Sq/Sk: lengths (varlen: maxima)
  int T;                      // query tokens
  int topk, nkb, tpc;         // key blocks per (b, kv head); tokens per chunk (128 / G)
  int causal;
  float scale_log2, cap_in, cap_out;
  int32_t* counts;       // [B * Hkv * nkb]
  int32_t* offsets;      // [B * Hkv * nkb + 1]
  int32_t* cursor;       // [B * Hkv * nkb]
  int32_t* chunkp;       // [B * Hkv * nkb + 1] prefix sums of chunks
  int32_t* entries;      // [T * Hkv * topk]: t * topk + slot, grouped by key block
  float* part_o;         // [topk, Bc, Sc, Hq, D]
  float* part_lse;       // [topk, Bc, Hq, Sc]
  int Bc, Sc;            // partial layout: (B, Sq) fixed length, (1, T) varlen
};

// Backward of block-sparse attention (fixed length, head dim 128).
struct BwdArgs {
  TensorArg q, k, v, o, dout;  // o may be bf16 or float32 (o_f32)
  int o_f32;
  const float* lse;            // [B, Hq, Sq] natural log (variable length: [Hq, total_q])
  float* dq;                   // [B, Sq, Hq, D] (variable length: [total_q, Hq, D]) float32, contiguous
  float* dk;                   // [B, Sk, Hkv, D] (variable length: [total_k, Hkv, D]) float32, contiguous
  float* dv;
  float* dsum;                 // sum_d dO * O, laid out as lse
  float* lse2;                 // lse in log2 units, +inf for a row with no keys (its weights are 0)
  PatternArg pat;              // kind 0 dense or 1 block lists
  const int32_t* cu_q;         // variable length: prefix sums of the query / key lengths, else null
  const int32_t* cu_k;
  int B, Hq, Hkv, G, Sq, Sk;   // Sq / Sk: lengths (variable length: maxima)
  int list_by_kv;
  int causal;
  float scale, scale_log2;
  float cap_in, cap_out;       // softcap constants (softcap_score); cap_in == 0: no softcap
  int BM;                      // query block rows of the pattern (64 or 128; dense: 128)
  int SB;                      // keys per sub-block (list): 32 per dK/dV wave, at most the pattern's block_N
  int nqb, nks;                // query blocks; sub-blocks
  int nkb, W;                  // pattern key blocks; bitmap words per (list head, key block)
  // per sub-block ("list"): its (query head, query block) pairs (block patterns), its units of
  // work (32-row query slabs), and those units cut into chunks of kBwdChunk
  int32_t* counts;             // [lists]: pairs (block patterns) or units (dense)
  int32_t* offsets;            // [lists + 1] prefix sums of pairs (block patterns)
  int32_t* entries;            // h * nqb + i
  int32_t* chunkp;             // [lists + 1] prefix sums of chunks
  uint32_t* bits;              // [B, Ht, nkb, W]: which query blocks name each key block
  float* part;                 // [chunks, 2, SB, D]: dK / dV partials of lists cut into chunks
};

struct ThresholdArgs {
  const float* tmax;  // [B, Hq, nqb, nqb] scaled tile maxima (j < i read)
  float* T;           // [Hq, nqb]
  int B, Hq, nqb, k;
};

struct CombineArgs {
  int P, B, Hq, Sq, D;
  const float* o_part;    // [P, B, Sq, Hq, D]
  const float* lse_part;  // [P, B, Hq, Sq]
  OutArg o;               // [B, Sq, Hq, D] view
  float* lse;             // [B, Hq, Sq] or nullptr
};

struct VSConvArgs {
  const int32_t* q_seqlens;
  const int32_t* kv_seqlens;
  const int32_t* vertical;  // [B, H, nnz_v]
  const int32_t* slash;     // [B, H, nnz_s]
  const int32_t* v_count;   // [H] valid vertical indices per head, or null (all nnz_v)
  const int32_t* s_count;   // [H] valid slash indices per head, or null (all nnz_s)
  int B, H, nnz_v, nnz_s, rows, BM, BN;
  int32_t* bc;              // [B, H, rows]
  int32_t* bo;              // [B, H, rows, nnz_s]
  int32_t* cc;              // [B, H, rows]
  int32_t* ci;              // [B, H, rows, nnz_v]
};

// Pattern contents check (check.cuh).
struct CheckArgs {
  PatternArg pat;
  const int32_t* cu_q;  // varlen prefix sums or null
  const int32_t* cu_k;
  int B, Ht, nqb, Sk;   // Sk: key length (fixed length)
  int32_t* result;      // [2]: violations, first violating list
};

}  // namespace bsa
