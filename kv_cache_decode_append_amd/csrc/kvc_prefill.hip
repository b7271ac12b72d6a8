// Chunked-prefill attention: write a prompt chunk's K/V into the paged cache,
// then causal attention of every chunk position over the cached prefix and the
// chunk's own positions up to itself.
//
// Prefill runs the prompt in parallel and is mostly matrix-matrix work
// (aiwithghost.com "KV cache and continuous batching: 1,000 people ask AI",
// section "What does a KV cache keep?"); it is capped at a fixed token budget
// per step so decode waits at most one chunk (gouthm.com "The KV cache is not
// your bottleneck", section "The fix that mattered"), and it can start after a
// prefix whose K/V are already cached (daviddominguez.dev "The KV cache and
// prefix caching", section "A prefix already in the cache can skip its
// prefill"). This is the one dense contraction of the path, so it runs on MFMA.
//
// Tiling (one workgroup = 4 waves = 128 query rows of one kv head):
//   row r <-> (position qt*MP + r / G, query head kvh*G + r % G), MP = 128 / G,
//   so the G query heads that share a K/V head share every K/V tile.
//   Keys are walked in tiles of 64 (four 16-token blocks through the block
//   table). Per tile and wave (2 row tiles of 16):
//     S^T[key][row] = K . Q^T          MFMA, A = K from LDS, B = Q from registers
//     online softmax per row            each lane owns one row (lane % 16)
//     O^T[dim][row] += V^T . P^T       MFMA, A = V^T from LDS, B = P from the S^T
//                                       registers (no transpose of P needed)
//   bf16: v_mfma_f32_16x16x32_bf16 (V staged transposed in LDS);
//   fp32: v_mfma_f32_16x16x4_f32 (V read row-major, one element per lane).
//   The reduction order inside an MFMA over keys is a permutation of the keys
//   (key 16m + 4g + i for lane group g); A and B use the same permutation.

#include <math.h>

#include "kvc_append.h"
#include "kvc_device.h"
#include "kvc_host.h"

namespace kvc {

constexpr int kPfWaves = 4;
constexpr int kRowTiles = 2;                        // 16-row tiles per wave
constexpr int kRows = kPfWaves * kRowTiles * 16;    // 128 query rows per workgroup
constexpr int kKeyTile = 64;                        // keys per staged tile

template <typename T> struct PfMfma;
template <> struct PfMfma<bf16_tag> {
  static constexpr int K = 32;                      // reduction depth per instruction
  using Frag = bf16x8_t;
  __device__ static f32x4 mma(const Frag& a, const Frag& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct PfMfma<float> {
  static constexpr int K = 4;
  using Frag = float;
  __device__ static f32x4 mma(const Frag& a, const Frag& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

template <typename T, int D, int G>
struct PfShape {
  static constexpr int EB = ElemBytes<T>::value;
  static constexpr int RB = D * EB;                 // bytes per K row in LDS
  static constexpr int NC = RB / 16;                // 16-byte chunks per row
  static constexpr int MP = kRows / G;              // positions per workgroup
  static constexpr int KS = D / PfMfma<T>::K;       // k-steps over head_dim
  static constexpr int DT = D / 16;                 // output dim tiles
  static constexpr bool BF16 = (EB == 2);
  static constexpr int VT_STRIDE = kKeyTile + 8;    // padded V^T row (elements), bf16 only
  static constexpr int K_LDS = kKeyTile * RB;
  static constexpr int V_LDS = BF16 ? D * VT_STRIDE * 2 : kKeyTile * RB;
  static constexpr int SMEM = K_LDS + V_LDS;
  static_assert(kRows % G == 0, "G divides 128");
};

struct PrefillArgs {
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* cu;
  const int32_t* prefix;
  const int32_t* bt;
  void* out;
  int32_t* err;
  int32_t hkv;
  int32_t num_blocks;
  int32_t max_blocks;
  int32_t total;
  int32_t max_chunk;
  float scale_log2;
};

template <typename T>
__device__ __forceinline__ void store4(void* out, size_t idx, const f32x4& v, float inv);
template <>
__device__ __forceinline__ void store4<float>(void* out, size_t idx, const f32x4& v, float inv) {
  *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + idx) =
      f32x4{v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv};
}
template <>
__device__ __forceinline__ void store4<bf16_tag>(void* out, size_t idx, const f32x4& v, float inv) {
  *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out) + idx) =
      u32x2{pack_bf16x2(v[0] * inv, v[1] * inv), pack_bf16x2(v[2] * inv, v[3] * inv)};
}

template <typename T, int D, int G>
__global__ __launch_bounds__(kPfWaves * 64) void prefill_attention_kernel(PrefillArgs a) {
  using S = PfShape<T, D, G>;
  using M = PfMfma<T>;
  using Frag = typename M::Frag;
  __shared__ __attribute__((aligned(16))) uint8_t smem[S::SMEM];
  uint8_t* k_lds = smem;
  uint8_t* v_lds = smem + S::K_LDS;

  const int qt = blockIdx.x, kvh = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int t0 = a.cu[s];
  const int C = a.cu[s + 1] - t0;
  const int p0 = a.prefix[s];
  const int pos_lo = qt * S::MP;
  if (!chunk_ok(t0, C, p0, a.total, a.max_chunk)) {
    if (qt == 0 && kvh == 0 && tid == 0) flag_error(a.err, KVC_DEVERR_CONTEXT);
    return;
  }
  if (pos_lo >= C) return;
  const int kv_len = p0 + C;                           // keys that exist after the write
  const int last_pos = p0 + min(pos_lo + S::MP, C) - 1;
  const int n_tiles = last_pos / kKeyTile + 1;
  const int hq_all = a.hkv * G;
  const int32_t* bt_row = a.bt + (size_t)s * a.max_blocks;

  // rows owned by this lane: r = w*32 + n*16 + l16
  int row_pos[kRowTiles];                              // absolute position (clamped)
  bool row_ok[kRowTiles];
  Frag qf[kRowTiles][S::KS];
#pragma unroll
  for (int n = 0; n < kRowTiles; ++n) {
    const int r = w * (kRowTiles * 16) + n * 16 + l16;
    const int pl = pos_lo + r / G, h = r % G;
    row_ok[n] = pl < C;
    row_pos[n] = p0 + min(pl, C - 1);
    const size_t qrow = ((size_t)(t0 + min(pl, C - 1)) * hq_all + kvh * G + h) * D;
#pragma unroll
    for (int kk = 0; kk < S::KS; ++kk) {
      if constexpr (S::BF16) {
        const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + qrow + kk * 32 + g * 8;
        qf[n][kk] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4*>(qp));
      } else {
        qf[n][kk] = reinterpret_cast<const float*>(a.q)[qrow + kk * 4 + g];
      }
    }
  }

  f32x4 o[kRowTiles][S::DT];
  float m_run[kRowTiles], l_run[kRowTiles];
#pragma unroll
  for (int n = 0; n < kRowTiles; ++n) {
    m_run[n] = -INFINITY;
    l_run[n] = 0.f;
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt) o[n][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.kc);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.vc);
  // byte offset of token `key` (row start) of this kv head, or -1 when absent
  auto row_off = [&](int key) -> int64_t {
    if (key >= kv_len) return -1;
    const int lb = key >> 4;
    if (lb >= a.max_blocks) {
      flag_error(a.err, KVC_DEVERR_CONTEXT);
      return -1;
    }
    const int blk = bt_row[lb];
    if ((unsigned)blk >= (unsigned)a.num_blocks) {
      flag_error(a.err, KVC_DEVERR_BLOCK_ID);
      return -1;
    }
    return (((int64_t)blk * a.hkv + kvh) * 16 + (key & 15)) * S::RB;
  };

  for (int kt = 0; kt < n_tiles; ++kt) {
    const int key0 = kt * kKeyTile;
    __syncthreads();                                   // previous tile fully consumed
    // ---- stage K (row-major, chunk-swizzled) ----
    for (int ci = tid; ci < kKeyTile * S::NC; ci += kPfWaves * 64) {
      const int key = ci / S::NC, c = ci % S::NC;
      const int64_t off = row_off(key0 + key);
      u32x4 val = u32x4{0u, 0u, 0u, 0u};
      if (off >= 0) val = *reinterpret_cast<const u32x4*>(kbase + off + c * 16);
      *reinterpret_cast<u32x4*>(k_lds + key * S::RB + ((c ^ (key % S::NC)) << 4)) = val;
    }
    // ---- stage V ----
    if constexpr (S::BF16) {
      // transposed: V^T[dim][key], rows padded to VT_STRIDE elements
      uint16_t* vt = reinterpret_cast<uint16_t*>(v_lds);
      for (int u = tid; u < (kKeyTile / 4) * S::NC; u += kPfWaves * 64) {
        const int kq = u / S::NC, c = u % S::NC;     // keys 4kq..4kq+3, dims 8c..8c+7
        u32x4 r4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t off = row_off(key0 + kq * 4 + j);
          r4[j] = u32x4{0u, 0u, 0u, 0u};
          if (off >= 0) r4[j] = *reinterpret_cast<const u32x4*>(vbase + off + c * 16);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int word = e >> 1, sh = (e & 1) * 16;
          uint32_t x[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) x[j] = (r4[j][word] >> sh) & 0xffffu;
          *reinterpret_cast<u32x2*>(vt + (c * 8 + e) * S::VT_STRIDE + kq * 4) =
              u32x2{x[0] | (x[1] << 16), x[2] | (x[3] << 16)};
        }
      }
    } else {
      for (int ci = tid; ci < kKeyTile * S::NC; ci += kPfWaves * 64) {
        const int key = ci / S::NC, c = ci % S::NC;
        const int64_t off = row_off(key0 + key);
        u32x4 val = u32x4{0u, 0u, 0u, 0u};
        if (off >= 0) val = *reinterpret_cast<const u32x4*>(vbase + off + c * 16);
        *reinterpret_cast<u32x4*>(v_lds + key * S::RB + ((c ^ (key % S::NC)) << 4)) = val;
      }
    }
    __syncthreads();

    // ---- S^T = K . Q^T : 4 key tiles x kRowTiles row tiles ----
    f32x4 sacc[4][kRowTiles];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int n = 0; n < kRowTiles; ++n) sacc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int key = m * 16 + l16;
#pragma unroll
      for (int kk = 0; kk < S::KS; ++kk) {
        Frag kf;
        if constexpr (S::BF16) {
          const int c = kk * 4 + g;
          kf = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4*>(
                                                k_lds + key * S::RB + ((c ^ (key % S::NC)) << 4)));
        } else {
          const int c = kk;                          // dims 4kk .. 4kk+3, element g
          kf = *reinterpret_cast<const float*>(k_lds + key * S::RB + ((c ^ (key % S::NC)) << 4) +
                                               g * 4);
        }
#pragma unroll
        for (int n = 0; n < kRowTiles; ++n) sacc[m][n] = M::mma(kf, qf[n][kk], sacc[m][n]);
      }
    }

    // ---- online softmax per row (lane owns row l16 of each row tile) ----
    const bool diag = key0 + kKeyTile - 1 > p0 + pos_lo;   // some key may pass some row
    float pbuf[4][kRowTiles][4];
#pragma unroll
    for (int n = 0; n < kRowTiles; ++n) {
      float mx = -INFINITY;
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = sacc[m][n][i];
          if (diag && key0 + m * 16 + g * 4 + i > row_pos[n]) v = -INFINITY;
          pbuf[m][n][i] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[n], mx * a.scale_log2);
      const float m_safe = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[n] - m_safe);
      float rs = 0.f;
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(pbuf[m][n][i], a.scale_log2, -m_safe));
          pbuf[m][n][i] = p;
          rs += p;
        }
      rs += __shfl_xor(rs, 16);
      rs += __shfl_xor(rs, 32);
      l_run[n] = l_run[n] * alpha + rs;
      m_run[n] = m_new;
#pragma unroll
      for (int dt = 0; dt < S::DT; ++dt) o[n][dt] *= alpha;
    }

    // ---- O^T += V^T . P^T ----
    if constexpr (S::BF16) {
      const uint16_t* vt = reinterpret_cast<const uint16_t*>(v_lds);
#pragma unroll
      for (int mp = 0; mp < 2; ++mp) {                 // key tiles (2mp, 2mp+1) = 32 keys
        Frag pf[kRowTiles];
#pragma unroll
        for (int n = 0; n < kRowTiles; ++n) {
          const float* a0 = pbuf[2 * mp][n];
          const float* a1 = pbuf[2 * mp + 1][n];
          const u32x4 pk = u32x4{pack_bf16x2(a0[0], a0[1]), pack_bf16x2(a0[2], a0[3]),
                                 pack_bf16x2(a1[0], a1[1]), pack_bf16x2(a1[2], a1[3])};
          pf[n] = __builtin_bit_cast(bf16x8_t, pk);
        }
#pragma unroll
        for (int dt = 0; dt < S::DT; ++dt) {
          const uint16_t* rowp = vt + (dt * 16 + l16) * S::VT_STRIDE + mp * 32 + g * 4;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(rowp);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(rowp + 16);
          const Frag vf = __builtin_bit_cast(bf16x8_t, u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
          for (int n = 0; n < kRowTiles; ++n) o[n][dt] = M::mma(vf, pf[n], o[n][dt]);
        }
      }
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = m * 16 + g * 4 + i;
#pragma unroll
          for (int dt = 0; dt < S::DT; ++dt) {
            const int dim = dt * 16 + l16, c = dim >> 2;
            const float vf = *reinterpret_cast<const float*>(
                v_lds + key * S::RB + ((c ^ (key % S::NC)) << 4) + (dim & 3) * 4);
#pragma unroll
            for (int n = 0; n < kRowTiles; ++n) o[n][dt] = M::mma(vf, pbuf[m][n][i], o[n][dt]);
          }
        }
    }
  }

  // ---- write rows: lane holds dims 16dt + 4g .. +3 of row l16 ----
#pragma unroll
  for (int n = 0; n < kRowTiles; ++n) {
    if (!row_ok[n]) continue;
    const int r = w * (kRowTiles * 16) + n * 16 + l16;
    const int pl = pos_lo + r / G, h = r % G;
    const size_t orow = ((size_t)(t0 + pl) * hq_all + kvh * G + h) * D;
    const float inv = 1.f / l_run[n];
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt) store4<T>(a.out, orow + dt * 16 + g * 4, o[n][dt], inv);
  }
}

template <typename T, int D, int G>
int launch_prefill(const PrefillArgs& a, int n_seqs, int max_chunk, hipStream_t st) {
  using S = PfShape<T, D, G>;
  const int n_qt = (max_chunk + S::MP - 1) / S::MP;
  hipLaunchKernelGGL((prefill_attention_kernel<T, D, G>), dim3(n_qt, a.hkv, n_seqs),
                     dim3(kPfWaves * 64), 0, st, a);
  return launch_status();
}

template <typename T, int D>
int prefill_g(const PrefillArgs& a, int G, int n, int mc, hipStream_t st) {
  switch (G) {
    case 1: return launch_prefill<T, D, 1>(a, n, mc, st);
    case 2: return launch_prefill<T, D, 2>(a, n, mc, st);
    case 4: return launch_prefill<T, D, 4>(a, n, mc, st);
    case 8: return launch_prefill<T, D, 8>(a, n, mc, st);
  }
  return KVC_ERR_UNSUPPORTED;
}

int dispatch_prefill(const PrefillArgs& a, int dtype, int D, int G, int n, int mc, hipStream_t st) {
  if (dtype == KVC_F32) {
    switch (D) {
      case 16: return prefill_g<float, 16>(a, G, n, mc, st);
      case 32: return prefill_g<float, 32>(a, G, n, mc, st);
      case 64: return prefill_g<float, 64>(a, G, n, mc, st);
      case 128: return prefill_g<float, 128>(a, G, n, mc, st);
    }
  } else {
    switch (D) {
      case 32: return prefill_g<bf16_tag, 32>(a, G, n, mc, st);
      case 64: return prefill_g<bf16_tag, 64>(a, G, n, mc, st);
      case 128: return prefill_g<bf16_tag, 128>(a, G, n, mc, st);
    }
  }
  return KVC_ERR_UNSUPPORTED;
}

}  // namespace kvc

extern "C" int kvc_chunked_prefill_attention(const kvc_cache* cache, const void* q, const void* k,
                                             const void* v, int32_t n_seqs, const int32_t* cu_chunk_lens,
                                             const int32_t* prefix_lens, int32_t total_tokens,
                                             int32_t max_chunk_len, const int32_t* block_table,
                                             int32_t max_blocks, int32_t Hq, float softmax_scale,
                                             void* out, void* stream) {
  int st = kvc::check_cache(cache);
  if (st != KVC_OK) return st;
  if (n_seqs < 0 || total_tokens < 0 || max_chunk_len < 0 || max_blocks < 0 || Hq <= 0)
    return KVC_ERR_SHAPE;
  if (Hq % cache->num_kv_heads != 0) return KVC_ERR_SHAPE;
  const int G = Hq / cache->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return KVC_ERR_UNSUPPORTED;
  if (n_seqs == 0 || total_tokens == 0 || max_chunk_len == 0) return KVC_OK;
  if (!q || !k || !v || !cu_chunk_lens || !prefix_lens || !block_table || !out) return KVC_ERR_NULL;
  hipStream_t s = kvc::as_stream(stream);
  st = kvc::launch_chunk_append(cache, k, v, n_seqs, cu_chunk_lens, prefix_lens, total_tokens,
                                max_chunk_len, block_table, max_blocks, s);
  if (st != KVC_OK) return st;
  kvc::PrefillArgs a;
  a.q = q;
  a.kc = cache->k_cache;
  a.vc = cache->v_cache;
  a.cu = cu_chunk_lens;
  a.prefix = prefix_lens;
  a.bt = block_table;
  a.out = out;
  a.err = cache->err_flag;
  a.hkv = cache->num_kv_heads;
  a.num_blocks = cache->num_blocks;
  a.max_blocks = max_blocks;
  a.total = total_tokens;
  a.max_chunk = max_chunk_len;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  return kvc::dispatch_prefill(a, cache->dtype, cache->head_dim, G, n_seqs, max_chunk_len, s);
}
