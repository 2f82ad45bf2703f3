// Attention over the compressed cache for gfx950 (CDNA4).
//
// Method: QuantWM reconstructs each Key as centre + dequantized 2-bit residual
// + U c_hat, the PSAC compensation applied at cache reconstruction ([digest]
// "Flickering after quantization? ...", PSAC paragraph); the review describes
// the same term as a low-rank correction of the attention logits
// ([review] summary).  The logits are the Query-Key dot products ([abstract]).
//
// Design.  A workgroup of 4 waves owns 128 queries of one head (32 per wave)
// and one key range (split-KV).  Per 64-key tile the workgroup rebuilds
//   K~ [64][d + 16 n] fp16 in LDS: mu_K[idx] + (z + code s) in fp32, rounded
//        once to fp16; the 16 n extra columns (n = 1 for r <= 16, 2 for
//        r <= 32) hold c_hat = coef * sigma,
//   V~^T [d][64] fp16 in LDS, keys permuted inside each 16-key chunk so that
//        the P^T operand can be taken straight from the S^T accumulators.
// Each wave computes S^T = K~ [Q | U^T q]^T with v_mfma_f32_32x32x16_f16
// (lane = query, 16 keys per 32-key block), so PSAC costs 16 n extra
// contraction columns instead of per-element work: q.(k_hat + U c_hat) =
// q.k_hat + (U^T q).c_hat.  Online softmax in base 2, then O^T += V~^T P^T.
#include "qwm_internal.h"

#include <hip/hip_fp16.h>

namespace qwm {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BN = 64;   // keys per tile
constexpr int BM = 128;  // queries per workgroup
constexpr float kLn2 = 0.6931471805599453f;

enum { MODE_ATTN = 0, MODE_LOGITS = 1, MODE_TOP1 = 2 };

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float h2f(uint16_t b) { return __half2float(__ushort_as_half(b)); }

template <bool F32IO>
__device__ __forceinline__ void load8f(const void* base, int64_t elem, float (&v)[8]) {
  if constexpr (F32IO) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
    float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
    v[0] = bf_lo(w.x); v[1] = bf_hi(w.x); v[2] = bf_lo(w.y); v[3] = bf_hi(w.y);
    v[4] = bf_lo(w.z); v[5] = bf_hi(w.z); v[6] = bf_lo(w.w); v[7] = bf_hi(w.w);
  }
}

__device__ __forceinline__ int load_idx(const void* base, int bytes, int64_t i) {
  return bytes == 1 ? (int)static_cast<const uint8_t*>(base)[i] : (int)static_cast<const uint16_t*>(base)[i];
}

// position of key k (0..15) of a 16-key chunk in the V~^T LDS rows
__device__ __forceinline__ int vperm(int k) { return 8 * ((k >> 2) & 1) + 4 * (k >> 3) + (k & 3); }

// NPS: 16-column PSAC k-steps (1 for r <= 16, 2 for r <= 32)
template <int D, bool F32IO, int MODE, int NPS>
__global__ __launch_bounds__(256) void attn_kernel(AttnParams p) {
  constexpr int DA = D + 16 * NPS; // contraction incl. the PSAC columns
  constexpr int KROW = DA + 8;     // fp16 pitch of K~ rows
  constexpr int VROW = BN + 8;     // fp16 pitch of V~^T rows
  constexpr int NKS = DA / 16;     // MFMA k-steps for S
  constexpr int NDB = D / 32;      // 32-row blocks of O^T
  constexpr int NG = D / 16;
  constexpr int CPT = D / 4;       // channels per thread in the tile rebuild
  constexpr int GPT = CPT / 16;    // residual groups per thread
  __shared__ __align__(16) _Float16 kt[BN * KROW];
  __shared__ __align__(16) _Float16 vt[MODE == MODE_TOP1 ? 8 : D * VROW];
  // fp32 activations keep the fp16 remainders of K~ and V~ as a second operand
  __shared__ __align__(16) _Float16 kt_lo[F32IO ? BN * KROW : 8];
  __shared__ __align__(16) _Float16 vt_lo[(F32IO && MODE != MODE_TOP1) ? D * VROW : 8];

  const int h = blockIdx.y;
  const int split = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hf = lane >> 5;
  const int l32 = lane & 31;
  const int qi = blockIdx.x * BM + wave * 32 + l32;
  const bool qvalid = qi < p.n_q;

  // ---- Q fragment [q | U^T q] as fp16, lane = query, half hf holds k-slots 8hf..8hf+7 ----
  half8 qf[NKS];
  half8 qlo[F32IO ? NG : 1];  // fp32 queries: the fp16 remainder q - fp16(q)
  {
    const void* qrow = F32IO
        ? static_cast<const void*>(static_cast<const float*>(p.q) + (int64_t)h * p.q_head_stride)
        : static_cast<const void*>(static_cast<const uint16_t*>(p.q) + (int64_t)h * p.q_head_stride);
    const int64_t qoff = (int64_t)(qvalid ? qi : 0) * p.q_token_stride;
    const float* U = p.u + (int64_t)h * D * p.r;
    float uq[16 * NPS];
#pragma unroll
    for (int i = 0; i < 16 * NPS; ++i) uq[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const int c0 = 16 * ks + 8 * hf;
      float v[8];
      if (qvalid) load8f<F32IO>(qrow, qoff + c0, v);
      else for (int i = 0; i < 8; ++i) v[i] = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        qf[ks][i] = (_Float16)v[i];
        if constexpr (F32IO) qlo[ks][i] = (_Float16)(v[i] - (float)qf[ks][i]);
#pragma unroll
        for (int rr = 0; rr < 16 * NPS; ++rr)
          if (rr < p.r) uq[rr] = fmaf(U[(c0 + i) * p.r + rr], v[i], uq[rr]);
      }
    }
#pragma unroll
    for (int i = 0; i < 16 * NPS; ++i) uq[i] += __shfl_xor(uq[i], 32);
    // PSAC k-step s: half hf holds directions 16s + 8hf .. 16s + 8hf + 7
#pragma unroll
    for (int s2 = 0; s2 < NPS; ++s2)
#pragma unroll
      for (int i = 0; i < 8; ++i) qf[NG + s2][i] = (_Float16)(hf ? uq[16 * s2 + 8 + i] : uq[16 * s2 + i]);
  }

  const int kbeg = split * p.keys_per_split;
  const int kend = min(p.n_k, kbeg + p.keys_per_split);

  float m_run = -INFINITY;  // running max (log2 units)
  float l_run = 0.f;        // this lane's partial sum
  f32x16 o[MODE == MODE_TOP1 ? 1 : NDB];
#pragma unroll
  for (int b = 0; b < (MODE == MODE_TOP1 ? 1 : NDB); ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[b][i] = 0.f;
  float best = -INFINITY;
  int best_k = 0x7fffffff;

  const void* muk = F32IO ? static_cast<const void*>(static_cast<const float*>(p.mu_k) + (int64_t)h * p.C_k * D)
                          : static_cast<const void*>(static_cast<const uint16_t*>(p.mu_k) + (int64_t)h * p.C_k * D);
  const void* muv = F32IO ? static_cast<const void*>(static_cast<const float*>(p.mu_v) + (int64_t)h * p.C_v * D)
                          : static_cast<const void*>(static_cast<const uint16_t*>(p.mu_v) + (int64_t)h * p.C_v * D);

  for (int t0 = kbeg; t0 < kend; t0 += BN) {
    __syncthreads();
    // ---- rebuild the tile: thread -> key kk, channel quarter qq ----
    {
      const int kk = threadIdx.x >> 2, qq = threadIdx.x & 3;
      const int key = t0 + kk;
      const bool kv = key < kend;
      const int64_t slot = (int64_t)h * p.Ncap + (kv ? key : 0);
      const int tile = (key / p.F) * p.tpf + (key % p.F) / p.T;
      const int64_t pslot = ((int64_t)h * p.Pcap + (kv ? tile : 0)) * NG;
      const int ck = kv ? min(load_idx(p.idx_k, p.idx_k_bytes, slot), p.C_k - 1) : 0;
#pragma unroll
      for (int gg = 0; gg < GPT; ++gg) {
        const int g = qq * GPT + gg;
        half8 out0, out1, lo0, lo1;
        if (kv) {
          const uint32_t w = p.codes_k[slot * NG + g];
          const uint32_t pz = p.params_k[pslot + g];
          const float z = h2f((uint16_t)(pz & 0xffff)), s = h2f((uint16_t)(pz >> 16));
          float m0[8], m1[8];
          load8f<F32IO>(muk, (int64_t)ck * D + 16 * g, m0);
          load8f<F32IO>(muk, (int64_t)ck * D + 16 * g + 8, m1);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float k0 = m0[j] + fmaf((float)((w >> (2 * j)) & 3u), s, z);
            const float k1 = m1[j] + fmaf((float)((w >> (2 * j + 16)) & 3u), s, z);
            out0[j] = (_Float16)k0;
            out1[j] = (_Float16)k1;
            if constexpr (F32IO) {
              lo0[j] = (_Float16)(k0 - (float)out0[j]);
              lo1[j] = (_Float16)(k1 - (float)out1[j]);
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            out0[j] = (_Float16)0.f; out1[j] = (_Float16)0.f;
            lo0[j] = (_Float16)0.f; lo1[j] = (_Float16)0.f;
          }
        }
        *reinterpret_cast<half8*>(&kt[kk * KROW + 16 * g]) = out0;
        *reinterpret_cast<half8*>(&kt[kk * KROW + 16 * g + 8]) = out1;
        if constexpr (F32IO) {
          *reinterpret_cast<half8*>(&kt_lo[kk * KROW + 16 * g]) = lo0;
          *reinterpret_cast<half8*>(&kt_lo[kk * KROW + 16 * g + 8]) = lo1;
        }
      }
      if (qq == 0) {
        float sg = 0.f;
        if (kv && p.r > 0) sg = h2f(p.coef_scale[slot]);
#pragma unroll
        for (int s2 = 0; s2 < NPS; ++s2) {
          half8 c0, c1;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int d0 = 16 * s2 + i, d1 = 16 * s2 + 8 + i;
            c0[i] = (_Float16)((kv && d0 < p.r) ? (float)p.coef[slot * p.r + d0] * sg : 0.f);
            c1[i] = (_Float16)((kv && d1 < p.r) ? (float)p.coef[slot * p.r + d1] * sg : 0.f);
          }
          *reinterpret_cast<half8*>(&kt[kk * KROW + D + 16 * s2]) = c0;
          *reinterpret_cast<half8*>(&kt[kk * KROW + D + 16 * s2 + 8]) = c1;
          if constexpr (F32IO) {
            half8 zz;
#pragma unroll
            for (int i = 0; i < 8; ++i) zz[i] = (_Float16)0.f;
            *reinterpret_cast<half8*>(&kt_lo[kk * KROW + D + 16 * s2]) = zz;
            *reinterpret_cast<half8*>(&kt_lo[kk * KROW + D + 16 * s2 + 8]) = zz;
          }
        }
      }
      if constexpr (MODE != MODE_TOP1) {
        const int cv = kv ? min(load_idx(p.idx_v, p.idx_v_bytes, slot), p.C_v - 1) : 0;
        const int col = (kk & ~15) + vperm(kk & 15);
#pragma unroll
        for (int gg = 0; gg < GPT; ++gg) {
          const int g = qq * GPT + gg;
          float vals[16];
          if (kv) {
            const uint32_t w = p.codes_v[slot * NG + g];
            const uint32_t pz = p.params_v[pslot + g];
            const float z = h2f((uint16_t)(pz & 0xffff)), s = h2f((uint16_t)(pz >> 16));
            float m0[8], m1[8];
            load8f<F32IO>(muv, (int64_t)cv * D + 16 * g, m0);
            load8f<F32IO>(muv, (int64_t)cv * D + 16 * g + 8, m1);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              vals[j] = m0[j] + fmaf((float)((w >> (2 * j)) & 3u), s, z);
              vals[8 + j] = m1[j] + fmaf((float)((w >> (2 * j + 16)) & 3u), s, z);
            }
          } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) vals[j] = 0.f;
          }
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const _Float16 hv = (_Float16)vals[j];
            vt[(16 * g + j) * VROW + col] = hv;
            if constexpr (F32IO) vt_lo[(16 * g + j) * VROW + col] = (_Float16)(vals[j] - (float)hv);
          }
        }
      }
    }
    __syncthreads();

    // ---- S^T = K~ Q'^T: lane = query, keys 32mb + 8(i/4) + 4hf + i%4 ----
    f32x16 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[mb][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const half8 a = *reinterpret_cast<const half8*>(&kt[(32 * mb + l32) * KROW + 16 * ks + 8 * hf]);
        s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[ks], s[mb], 0, 0, 0);
        if constexpr (F32IO) {
          if (ks < NG) {
            s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qlo[ks], s[mb], 0, 0, 0);
            const half8 al = *reinterpret_cast<const half8*>(&kt_lo[(32 * mb + l32) * KROW + 16 * ks + 8 * hf]);
            s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, qf[ks], s[mb], 0, 0, 0);
          }
        }
      }
    }

    if constexpr (MODE == MODE_TOP1) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = t0 + 32 * mb + 8 * (i / 4) + 4 * hf + (i % 4);
          const float v = s[mb][i];
          if (key < kend && (v > best || (v == best && key < best_k))) { best = v; best_k = key; }
        }
      continue;
    } else {
      // ---- online softmax (base 2) ----
      float mt = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = t0 + 32 * mb + 8 * (i / 4) + 4 * hf + (i % 4);
          float t = s[mb][i] * p.scale_log2;
          if (key >= kend) t = -INFINITY;
          if constexpr (MODE == MODE_LOGITS) {
            if (qvalid && key < kend)
              p.logits[((int64_t)h * p.n_q + qi) * p.n_k + key] = s[mb][i] * p.scale;
          }
          s[mb][i] = t;
          mt = fmaxf(mt, t);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float m_new = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      float psum = 0.f;
      half8 pf[4];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = __builtin_amdgcn_exp2f(s[mb][i] - m_new);
          psum += e;
          pf[2 * mb + i / 8][i % 8] = (_Float16)e;
        }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int b = 0; b < NDB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[b][i] *= alpha;
      // ---- O^T += V~^T P^T ----
#pragma unroll
      for (int b = 0; b < NDB; ++b)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const half8 a = *reinterpret_cast<const half8*>(&vt[(32 * b + l32) * VROW + 16 * c + 8 * hf]);
          o[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[c], o[b], 0, 0, 0);
          if constexpr (F32IO) {
            const half8 al = *reinterpret_cast<const half8*>(&vt_lo[(32 * b + l32) * VROW + 16 * c + 8 * hf]);
            o[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, pf[c], o[b], 0, 0, 0);
          }
        }
    }
  }

  if constexpr (MODE == MODE_TOP1) {
    const float ob = __shfl_xor(best, 32);
    const int ok = __shfl_xor(best_k, 32);
    if (ob > best || (ob == best && ok < best_k)) { best = ob; best_k = ok; }
    if (qvalid && hf == 0) p.top1[(int64_t)h * p.n_q + qi] = best_k;
    return;
  } else if constexpr (MODE == MODE_LOGITS) {
    return;  // the debug variant only exports the logits
  } else {
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float lse = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    if (!qvalid) return;
    if (p.splits == 1) {
      if (p.lse && hf == 0) p.lse[(int64_t)h * p.n_q + qi] = lse;
      const int64_t obase = (int64_t)h * p.o_head_stride + (int64_t)qi * p.o_token_stride;
#pragma unroll
      for (int b = 0; b < NDB; ++b)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d0 = 32 * b + 8 * i4 + 4 * hf;
          if constexpr (F32IO) {
            float4 v = make_float4(o[b][4 * i4] * inv, o[b][4 * i4 + 1] * inv, o[b][4 * i4 + 2] * inv, o[b][4 * i4 + 3] * inv);
            *reinterpret_cast<float4*>(static_cast<float*>(p.out) + obase + d0) = v;
          } else {
            uint2 w;
            const __bf16 b0 = (__bf16)(o[b][4 * i4] * inv), b1 = (__bf16)(o[b][4 * i4 + 1] * inv);
            const __bf16 b2 = (__bf16)(o[b][4 * i4 + 2] * inv), b3 = (__bf16)(o[b][4 * i4 + 3] * inv);
            w.x = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
            w.y = (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + obase + d0) = w;
          }
        }
    } else {
      const int64_t pb = ((int64_t)split * gridDim.y + h) * p.n_q + qi;
      if (hf == 0) p.part_ml[pb] = lse;
#pragma unroll
      for (int b = 0; b < NDB; ++b)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d0 = 32 * b + 8 * i4 + 4 * hf;
          float4 v = make_float4(o[b][4 * i4] * inv, o[b][4 * i4 + 1] * inv, o[b][4 * i4 + 2] * inv, o[b][4 * i4 + 3] * inv);
          *reinterpret_cast<float4*>(p.part_o + pb * D + d0) = v;
        }
    }
  }
}

// Merge split-KV partials: o = sum_s exp(lse_s - lse) o_s, lse = log sum exp lse_s.
template <int D, bool F32IO>
__global__ __launch_bounds__(D) void combine_kernel(AttnParams p, int heads) {
  const int qi = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
  float top = -INFINITY;
  for (int s = 0; s < p.splits; ++s) top = fmaxf(top, p.part_ml[((int64_t)s * heads + h) * p.n_q + qi]);
  float tot = 0.f, acc = 0.f;
  if (top != -INFINITY) {
    for (int s = 0; s < p.splits; ++s) {
      const int64_t pb = ((int64_t)s * heads + h) * p.n_q + qi;
      const float w = __expf(p.part_ml[pb] - top);
      tot += w;
      acc += w * p.part_o[pb * D + d];
    }
  }
  const float o = tot > 0.f ? acc / tot : 0.f;
  const int64_t oi = (int64_t)h * p.o_head_stride + (int64_t)qi * p.o_token_stride + d;
  if constexpr (F32IO) static_cast<float*>(p.out)[oi] = o;
  else static_cast<__bf16*>(p.out)[oi] = (__bf16)o;
  if (d == 0 && p.lse) p.lse[(int64_t)h * p.n_q + qi] = tot > 0.f ? top + __logf(tot) : -INFINITY;
}

template <int D, bool F32IO, int NPS>
hipError_t launch_dn(const AttnParams& p, int heads, hipStream_t stream) {
  dim3 grid((p.n_q + BM - 1) / BM, heads, p.splits);
  if (p.ev_begin) {
    const hipError_t er = hipEventRecord(static_cast<hipEvent_t>(p.ev_begin), stream);
    if (er != hipSuccess) return er;
  }
  if (p.top1) {
    hipLaunchKernelGGL((attn_kernel<D, F32IO, MODE_TOP1, NPS>), grid, dim3(256), 0, stream, p);
  } else if (p.logits) {
    hipLaunchKernelGGL((attn_kernel<D, F32IO, MODE_LOGITS, NPS>), grid, dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL((attn_kernel<D, F32IO, MODE_ATTN, NPS>), grid, dim3(256), 0, stream, p);
  }
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && p.ev_end) e = hipEventRecord(static_cast<hipEvent_t>(p.ev_end), stream);
  if (e != hipSuccess || p.splits == 1 || p.top1 || p.logits) return e;
  return launch_combine(p, heads, D, F32IO, stream);
}

template <int D, bool F32IO>
hipError_t launch_d(const AttnParams& p, int heads, hipStream_t stream) {
  return p.r > 16 ? launch_dn<D, F32IO, 2>(p, heads, stream) : launch_dn<D, F32IO, 1>(p, heads, stream);
}

// Top-1 over original keys: one thread per (head, query), fp32 dot products.
template <int D, bool F32IO>
__global__ __launch_bounds__(256) void dense_top1_kernel(const void* q, int64_t qhs, int64_t qts, int n_q,
                                                         const void* k, int64_t khs, int64_t kts, int n_k,
                                                         int* top1) {
  const int h = blockIdx.y;
  const int qi = blockIdx.x * 256 + threadIdx.x;
  if (qi >= n_q) return;
  float qv[D];
  const void* qb = F32IO ? static_cast<const void*>(static_cast<const float*>(q) + (int64_t)h * qhs)
                         : static_cast<const void*>(static_cast<const uint16_t*>(q) + (int64_t)h * qhs);
  const void* kb = F32IO ? static_cast<const void*>(static_cast<const float*>(k) + (int64_t)h * khs)
                         : static_cast<const void*>(static_cast<const uint16_t*>(k) + (int64_t)h * khs);
#pragma unroll
  for (int j8 = 0; j8 < D / 8; ++j8) {
    float v[8];
    load8f<F32IO>(qb, (int64_t)qi * qts + 8 * j8, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) qv[8 * j8 + i] = v[i];
  }
  float best = -INFINITY;
  int bk = 0;
  for (int t = 0; t < n_k; ++t) {
    float acc = 0.f;
#pragma unroll
    for (int j8 = 0; j8 < D / 8; ++j8) {
      float v[8];
      load8f<F32IO>(kb, (int64_t)t * kts + 8 * j8, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc = fmaf(qv[8 * j8 + i], v[i], acc);
    }
    if (acc > best) { best = acc; bk = t; }
  }
  top1[(int64_t)h * n_q + qi] = bk;
}

}  // namespace

hipError_t launch_combine(const AttnParams& p, int heads, int head_dim, bool f32io, hipStream_t stream) {
  const dim3 grid(p.n_q, heads);
  if (head_dim == 128) {
    if (f32io) hipLaunchKernelGGL((combine_kernel<128, true>), grid, dim3(128), 0, stream, p, heads);
    else hipLaunchKernelGGL((combine_kernel<128, false>), grid, dim3(128), 0, stream, p, heads);
  } else {
    if (f32io) hipLaunchKernelGGL((combine_kernel<64, true>), grid, dim3(64), 0, stream, p, heads);
    else hipLaunchKernelGGL((combine_kernel<64, false>), grid, dim3(64), 0, stream, p, heads);
  }
  return hipGetLastError();
}

hipError_t launch_attention(const AttnParams& p, int heads, int head_dim, bool f32io, hipStream_t stream) {
  // bf16 activations: their own kernel, whose logits / top-1 exports are
  // compile-time variants of the same tile loop; fp32 activations: the
  // generic kernel
  if (!f32io) return launch_attention_bf16(p, heads, head_dim, stream);
  if (head_dim == 128) return f32io ? launch_d<128, true>(p, heads, stream) : launch_d<128, false>(p, heads, stream);
  return f32io ? launch_d<64, true>(p, heads, stream) : launch_d<64, false>(p, heads, stream);
}

hipError_t launch_dense_top1(const void* q, int64_t qhs, int64_t qts, int n_q, const void* k, int64_t khs,
                             int64_t kts, int n_k, int heads, int head_dim, bool f32io, int* top1,
                             hipStream_t stream) {
  dim3 grid((n_q + 255) / 256, heads);
  if (head_dim == 128) {
    if (f32io) hipLaunchKernelGGL((dense_top1_kernel<128, true>), grid, dim3(256), 0, stream, q, qhs, qts, n_q, k, khs, kts, n_k, top1);
    else hipLaunchKernelGGL((dense_top1_kernel<128, false>), grid, dim3(256), 0, stream, q, qhs, qts, n_q, k, khs, kts, n_k, top1);
  } else {
    if (f32io) hipLaunchKernelGGL((dense_top1_kernel<64, true>), grid, dim3(256), 0, stream, q, qhs, qts, n_q, k, khs, kts, n_k, top1);
    else hipLaunchKernelGGL((dense_top1_kernel<64, false>), grid, dim3(256), 0, stream, q, qhs, qts, n_q, k, khs, kts, n_k, top1);
  }
  return hipGetLastError();
}

}  // namespace qwm
