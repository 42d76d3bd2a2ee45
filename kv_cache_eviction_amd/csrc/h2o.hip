// H2O decode step on a preallocated slot cache.
//
// H2O ("H2O: Heavy-Hitter Oracle"), 3.4 and System Implementation Details:
// the new token's key/value go into a free slot of a preallocated cache (an
// evicted slot is overwritten in place, no data moves); the new query attends
// over the retained tokens and itself, o_i = softmax over the retained set
// (Def. 2.2); its probabilities are added to the per-slot accumulators
// (o~_i = o~_{i-1} + o_i); if the cache exceeds k_heavy + k_recent, the
// retained token outside the recent window with the lowest accumulated score
// is evicted (later position first on ties), at most one per step
// (Def. 2.1).  Rows (sequence, head) are independent, one wavefront each.
//
// A row's slots are read as 16-byte lane chunks, D/EPC lanes per slot, so one
// wave instruction covers 64*16 contiguous-per-slot bytes, and eight such
// instructions are in flight before any is used; invalid slots (and slots
// whose probability is 0 in the P.V pass) are never read: their loads take an
// offset past the buffer resource's range, which returns zeros without a
// memory access.  The slot map and the logits sit in LDS for the softmax; the
// updated accumulators are read back (same lane) for the arg-min.
#include "common.hpp"
#include "launch.hpp"
#include "timing.hpp"

namespace kvs {

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Sum over each group of LPR consecutive lanes (LPR a power of two <= 64),
// and over the lanes l, l + LPR, l + 2 LPR, ... : DPP within 16-lane rows,
// permlane swaps across them, no LDS traffic.
template <int LPR> __device__ __forceinline__ float lane_group_sum(float v) {
  if (LPR >= 2) v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
  if (LPR >= 4) v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
  if (LPR >= 8) v += dpp_f32<0x141>(v);  // row_half_mirror
  if (LPR >= 16) v += dpp_f32<0x140>(v); // row_mirror
  if (LPR >= 32) v = sum_xor16(v);
  if (LPR >= 64) v = sum_xor32(v);
  return v;
}
template <int LPR> __device__ __forceinline__ float across_groups_sum(float v) {
  if (LPR <= 8) v = sum_xor8(v);
  if (LPR <= 16) v = sum_xor16(v);
  if (LPR <= 32) v = sum_xor32(v);
  return v;
}

__device__ __forceinline__ uint32_t order_key_pos(float x) {
  const uint32_t u = __float_as_uint(x + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <typename T, int D>
__global__ void __launch_bounds__(256)
h2o_decode_kernel(const T *__restrict__ q, T *__restrict__ K, T *__restrict__ V,
                  const T *__restrict__ k_new, const T *__restrict__ v_new,
                  int32_t *__restrict__ slot_pos, float *__restrict__ acc, T *__restrict__ O,
                  int32_t *__restrict__ evict_slot, int rows, int cap, int cur_len, int k_heavy,
                  int k_recent, float c) {
  constexpr int EPC = 16 / (int)sizeof(T);
  constexpr int LPR = D / EPC;  // lanes per slot row
  constexpr int RPI = 64 / LPR; // slot rows per wave step
  constexpr int U = 8;          // wave steps whose loads are in flight together
  extern __shared__ float dsh[];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const long row = (long)blockIdx.x * 4 + wv;
  if (row >= rows) return;
  float *prob = dsh + (long)wv * 2 * cap;
  int32_t *pos_s = reinterpret_cast<int32_t *>(prob + cap);
  int32_t *pos = slot_pos + row * cap;
  float *ac = acc + row * cap;
  T *Kr = K + row * cap * D;
  T *Vr = V + row * cap * D;
  const uint32_t row_bytes = (uint32_t)cap * (uint32_t)(D * sizeof(T));
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kr, row_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vr, row_bytes);

  // slot map into LDS; lowest free slot, and how many slots hold a token
  int ws = -1, nvalid = 0;
  for (int base = 0; base < cap; base += 64) {
    const int s = base + lane;
    const int p = s < cap ? pos[s] : 0;
    if (s < cap) pos_s[s] = p;
    const unsigned long long fb = __ballot(s < cap && p < 0);
    const unsigned long long vb = __ballot(s < cap && p >= 0);
    nvalid += __popcll(vb);
    if (ws < 0 && fb) ws = base + __ffsll((long long)fb) - 1;
  }
  if (ws < 0) {
    if (lane == 0 && evict_slot) evict_slot[row] = -2;
    return;
  }
  wave_lds_sync();
  const int newpos = cur_len - 1;
  const int sub = lane % LPR, rr = lane / LPR;

  float qv[EPC], kn[EPC], vn[EPC];
  {
    const U128 qq = *reinterpret_cast<const U128 *>(q + row * D + sub * EPC);
    const U128 kk = *reinterpret_cast<const U128 *>(k_new + row * D + sub * EPC);
    const U128 vv = *reinterpret_cast<const U128 *>(v_new + row * D + sub * EPC);
    const T *qe = reinterpret_cast<const T *>(&qq);
    const T *ke = reinterpret_cast<const T *>(&kk);
    const T *ve = reinterpret_cast<const T *>(&vv);
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      qv[e] = to_f32(qe[e]);
      kn[e] = to_f32(ke[e]);
      vn[e] = to_f32(ve[e]);
    }
  }

  // logits of every valid slot (the new token's from registers); U wave steps
  // of K rows are loaded before any is used
  for (int base = 0; base < cap; base += RPI * U) {
    U128 kk[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = base + u * RPI + rr;
      const bool ld = s < cap && s != ws && pos_s[s] >= 0;
      kk[u] = buf_load16(rk, ld ? (uint32_t)(s * D + sub * EPC) * (uint32_t)sizeof(T) : kNoLoad);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = base + u * RPI + rr;
      const bool inb = s < cap;
      const bool valid = inb && (s == ws || pos_s[s] >= 0);
      const T *ke = reinterpret_cast<const T *>(&kk[u]);
      float part = 0.f;
      if (inb && s == ws) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) part += qv[e] * kn[e];
      } else {
#pragma unroll
        for (int e = 0; e < EPC; ++e) part += qv[e] * to_f32(ke[e]);
      }
      part = lane_group_sum<LPR>(part);
      if (sub == 0 && inb) prob[s] = valid ? part * c : -INFINITY;
    }
  }
  wave_lds_sync();

  float mx = -INFINITY;
  for (int s = lane; s < cap; s += 64) mx = fmaxf(mx, prob[s]);
  mx = wave_max_dpp(mx);
  float l = 0.f;
  for (int s = lane; s < cap; s += 64) l += hw_exp2(prob[s] - mx);
  l = wave_sum_dpp(l);
  const float inv = 1.f / l;
  for (int s = lane; s < cap; s += 64) {
    const bool valid = (s == ws) || pos_s[s] >= 0;
    float a = 0.f;
    if (valid) {
      a = hw_exp2(prob[s] - mx) * inv;
      ac[s] = ((s == ws) ? 0.f : ac[s]) + a;  // read back by this same lane below
    }
    prob[s] = a;
  }
  wave_lds_sync();

  if (O) {
    float ov[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) ov[e] = 0.f;
    for (int base = 0; base < cap; base += RPI * U) {
      U128 vv[U];
      float av[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int s = base + u * RPI + rr;
        av[u] = s < cap ? prob[s] : 0.f;
        const bool ld = av[u] != 0.f && s != ws;
        vv[u] = buf_load16(rv, ld ? (uint32_t)(s * D + sub * EPC) * (uint32_t)sizeof(T) : kNoLoad);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int s = base + u * RPI + rr;
        const T *ve = reinterpret_cast<const T *>(&vv[u]);
        if (s == ws) {
#pragma unroll
          for (int e = 0; e < EPC; ++e) ov[e] += av[u] * vn[e];
        } else {
#pragma unroll
          for (int e = 0; e < EPC; ++e) ov[e] += av[u] * to_f32(ve[e]);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < EPC; ++e) ov[e] = across_groups_sum<LPR>(ov[e]);
    if (rr == 0) {
      U128 out;
      T *oe = reinterpret_cast<T *>(&out);
#pragma unroll
      for (int e = 0; e < EPC; ++e) oe[e] = from_f32<T>(ov[e]);
      *reinterpret_cast<U128 *>(O + row * D + sub * EPC) = out;
    }
  }

  // the new token takes its slot
  if (rr == 0) {
    *reinterpret_cast<U128 *>(Kr + (long)ws * D + sub * EPC) =
        *reinterpret_cast<const U128 *>(k_new + row * D + sub * EPC);
    *reinterpret_cast<U128 *>(Vr + (long)ws * D + sub * EPC) =
        *reinterpret_cast<const U128 *>(v_new + row * D + sub * EPC);
  }
  if (lane == 0) pos[ws] = newpos;

  int ev = -1;
  if (nvalid + 1 > k_heavy + k_recent) {
    const int recent_from = cur_len - k_recent;
    unsigned long long best = ~0ull;
    for (int s = lane; s < cap; s += 64) {
      const int p = (s == ws) ? newpos : pos_s[s];
      if (p >= 0 && p < recent_from) {
        const unsigned long long key =
            ((unsigned long long)order_key_pos(ac[s]) << 32) | (uint32_t)(0x7FFFFFFF - p);
        best = key < best ? key : best;
      }
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const unsigned long long other = __shfl_xor(best, o, 64);
      best = other < best ? other : best;
    }
    if (best != ~0ull) {
      const int pev = 0x7FFFFFFF - (int)(uint32_t)(best & 0xFFFFFFFFull);
      int cand = -1;
      for (int s = lane; s < cap; s += 64) {
        const int p = (s == ws) ? newpos : pos_s[s];
        if (p == pev) cand = s;
      }
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) cand = max(cand, __shfl_xor(cand, o, 64));
      ev = cand;
    }
  }
  if (lane == 0) {
    if (ev >= 0) pos[ev] = -1;
    if (evict_slot) evict_slot[row] = ev;
  }
}

template <typename T, int D>
static hipError_t run_decode(int rows, int cap, int cur_len, int k_heavy, int k_recent,
                             const void *q, void *K, void *V, const void *k_new,
                             const void *v_new, int32_t *slot_pos, float *acc, void *O,
                             int32_t *evict_slot, hipStream_t st) {
  const float c = kLog2e / sqrtf((float)D);
  const size_t shm = sizeof(float) * 2 * (size_t)cap * 4;  // probabilities and slot map per wave
  {
    TimedLaunch tl_("h2o_decode", st);
    hipLaunchKernelGGL((h2o_decode_kernel<T, D>), dim3((rows + 3) / 4), dim3(256), shm, st,
                       (const T *)q, (T *)K, (T *)V, (const T *)k_new, (const T *)v_new, slot_pos,
                       acc, (T *)O, evict_slot, rows, cap, cur_len, k_heavy, k_recent, c);
  }
  return hipGetLastError();
}

hipError_t launch_h2o_decode(int etype, int d, int rows, int cap, int cur_len, int k_heavy,
                             int k_recent, const void *q, void *K, void *V, const void *k_new,
                             const void *v_new, int32_t *slot_pos, float *acc, void *O,
                             int32_t *evict_slot, hipStream_t st) {
#define KVS_D(T, DD)                                                                          \
  return run_decode<T, DD>(rows, cap, cur_len, k_heavy, k_recent, q, K, V, k_new, v_new,     \
                           slot_pos, acc, O, evict_slot, st)
  if (etype == E_F32) { if (d == 64) KVS_D(float, 64); KVS_D(float, 128); }
  if (etype == E_BF16) { if (d == 64) KVS_D(bf16, 64); KVS_D(bf16, 128); }
  if (d == 64) KVS_D(f16, 64);
  KVS_D(f16, 128);
#undef KVS_D
}

}  // namespace kvs
