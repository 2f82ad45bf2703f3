// Internal declarations shared by the host library and the HIP kernels.
// Not part of the public ABI (include/qwm.h); symbols are hidden.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define QWM_HIDDEN __attribute__((visibility("hidden")))

namespace qwm {

// Tokens of one segment: a run of at most 32 tokens of one frame, starting at
// a multiple of 32 inside the frame.  Parameter tiles (T | 32) never straddle
// a segment.
constexpr int kSegTokens = 32;
constexpr int kSegsPerWave = 2;          // one 32-token MFMA N-block each
// centre rows staged for the screen: C rounded up to whole pairs of 32-centre blocks
inline int append_cpad(int C) { return (C + 63) / 64 * 64; }

struct AppendParams {
  // input activations [H][n_new][d]
  const void* x;
  int64_t head_stride, token_stride;  // elements
  int n_new;
  int frame0;          // global frame index of the first appended frame
  int F, T, tpf;       // frame tokens, group tokens, tiles per frame
  int segs_per_frame;  // ceil(F / 32)
  int total_segs;      // (n_new / F) * segs_per_frame
  int C, Cpad;         // centres (padded to a multiple of 64: an even number of 32-centre blocks)
  int Kc;              // tracked candidates: K_c for QSAC, 1 for argmin modes
  int use_range;       // QSAC stage 2 active
  int s2mode;          // stage-2 score: 0 range model, 1 exact error (diagonal), 2 exact error (full M)
  int uniform;         // s = 1
  int r;               // PSAC rank (Keys); 0 for Values
  int64_t Ncap, Pcap;  // token / tile capacity per head
  // calibration (per-head arrays; the kernel adds the head offset)
  const void* mu;         // [H][C][d] io dtype
  const float* sens;      // [H][d]
  const double* u64;      // [H][d][RP] zero-padded
  int rp;                 // RP (row pitch of u64)
  const double* sgroup;   // [H][d/16]
  const double* moment;   // [H][d][d] full Query second moment (s2mode 2)
  const float* norm_half; // [H][C]  ||mu||^2/2 (weighted or not)
  const float* head_max;  // [H][4]
  int head_max_slot;
  // outputs (cache arrays, base of head 0)
  void* idx;
  int idx_bytes;
  uint32_t* codes;   // [H][Ncap][d/16]
  uint32_t* params;  // [H][Pcap][d/16] half2
  int8_t* coef;      // [H][Ncap][r]
  uint16_t* coef_scale;  // [H][Ncap] fp16 bits
  int64_t tok0;      // first cache token index of this append
  // optional path counters (device, uint32[4], nullable): tokens whose
  // candidate set was settled by exact rescoring of the screen's uncertain
  // band, and tokens that searched all centres; [0], [1] for Keys, [2], [3]
  // for Values
  uint32_t* counters;
};

// Attention over the compressed cache.
struct AttnParams {
  const void* q;
  int64_t q_head_stride, q_token_stride;
  int n_q;
  int n_k;
  int F, T, tpf;
  int r, rp;
  float scale_log2;  // softmax scale * log2(e)
  float scale;       // softmax scale
  int64_t Ncap, Pcap;
  int C_k, C_v;
  const void* mu_k;   // [H][C_K][d]
  const void* mu_v;   // [H][C_V][d]
  const float* u;     // [H][d][r] fp32
  const void* idx_k; int idx_k_bytes;
  const uint32_t* codes_k;
  const uint32_t* params_k;
  const int8_t* coef;
  const uint16_t* coef_scale;
  const void* idx_v; int idx_v_bytes;
  const uint32_t* codes_v;
  const uint32_t* params_v;
  // bf16 path: fp16 centres and U^T in paired channel order, and the
  // frame division key / F = (key + umulhi(key, divF_lo)) >> divF_s
  const uint16_t* mu_k16;  // [H][C_K][d]
  const uint16_t* mu_v16;  // [H][C_V][d]
  const uint16_t* ut16;    // [H][16][d]
  uint32_t divF_lo;
  int divF_s;
  int log2T;
  // optional local chunk (bf16 path): the current chunk's own uncompressed
  // Keys and Values [H][n_loc][d], attended together with the cache
  const void* k_loc;
  const void* v_loc;
  int64_t kl_head_stride, kl_token_stride, vl_head_stride, vl_token_stride;
  int n_loc;
  // outputs
  void* out;
  int64_t o_head_stride, o_token_stride;
  float* lse;            // [H][n_q] or null
  float* logits;         // debug [H][n_q][n_k] or null
  int* top1;             // measure [H][n_q] or null
  // optional HIP events recorded on the stream around the main attention
  // kernel (its combine pass excluded), for per-kernel timing
  void* ev_begin;
  void* ev_end;
  // split-KV partials
  int splits;            // number of key ranges
  int keys_per_split;    // multiple of the key tile
  float* part_o;         // [splits][H][n_q][d] fp32 (bf16 path: [slots][rows][d] fp16)
  float* part_ml;        // [splits][H][n_q] (bf16 path: [slots][rows]) natural-log lse
};

// Parts of the key axis of one attention call: compressed caches (epochs,
// each with its own calibration), then optionally the local chunk.  Each part
// starts at a tile boundary; a part's keys run from 0 to n_k in its own cache.
// Every part has the same configuration, so the fields sit at the same byte
// offsets inside each cache block and each calibration block.
constexpr int kMaxParts = 64;
struct CachePart {
  const unsigned char* cache;  // cache block
  const unsigned char* calib;  // its calibration block
  int n_k;                     // tokens of the part
  int tile0;                   // its first key tile
};
struct PartTable {
  CachePart part[kMaxParts];
  int n_parts;  // compressed parts (tiles from local0 on are the local chunk's)
  int local0;
  // byte offsets in the cache block, then in the calibration block
  int64_t idx_k, idx_v, codes_k, codes_v, params_k, params_v, coef, coef_scale;
  int64_t mu_k16, mu_v16, ut16;
};

QWM_HIDDEN hipError_t launch_append(const AppendParams& p, int heads, int head_dim, bool f32io,
                                    bool key, hipStream_t stream);
// Keys and Values of the same frames in one launch (pk, pv as for launch_append)
QWM_HIDDEN hipError_t launch_append_kv(const AppendParams& pk, const AppendParams& pv, int heads, int head_dim,
                                       bool f32io, hipStream_t stream);
QWM_HIDDEN hipError_t launch_attention(const AttnParams& p, int heads, int head_dim, bool f32io,
                                       hipStream_t stream);
// bf16 activations: softmax attention, or (p.logits / p.top1 set) the logits
// or top-1 export of the same kernel; with a part table (several compressed
// caches and / or the local chunk: p.n_loc), the key axis runs through the
// parts in order
QWM_HIDDEN hipError_t launch_attention_bf16(const AttnParams& p, int heads, int head_dim, hipStream_t stream,
                                            const PartTable* parts = nullptr);
QWM_HIDDEN hipError_t launch_combine(const AttnParams& p, int heads, int head_dim, bool f32io, hipStream_t stream);
// queries per workgroup of the bf16 attention kernel, and its workgroup cap
// (one per CU of the MI355X); the partial-result workspace holds two slots of
// kAttnBf16Queries rows per workgroup
constexpr int kAttnBf16Queries = 256;
constexpr int kAttnBf16MaxWorkgroups = 256;
QWM_HIDDEN hipError_t launch_dense_top1(const void* q, int64_t qhs, int64_t qts, int n_q,
                                        const void* k, int64_t khs, int64_t kts, int n_k,
                                        int heads, int head_dim, bool f32io, int* top1,
                                        hipStream_t stream);
QWM_HIDDEN size_t append_lds_bytes(int Cpad, int head_dim, bool f32io, int ucols, int waves);

}  // namespace qwm
