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
// wave instruction covers 64*16 contiguous-per-slot bytes.  Loads go in
// batches of eight such instructions, all in flight before the first is used
// (the first value batch is in flight while the softmax runs); free
// slots are never read: their loads take an offset past the buffer
// resource's range, which returns zeros without a memory access.  The slot
// map and accumulators are loaded once into LDS beside the logits, so the
// softmax, the accumulation and the arg-min touch global memory only to write.
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

// c + a * b for one 16-byte chunk of fp16 in each of a and b (the new query
// and a key row), elementwise in order, or c + a * b[e] for a scalar a and
// each element of b (a probability and a value row).  fp16 chunks feed the
// mixed-precision FMA straight from their packed registers: the product and
// sum are those of fp32, and no unpacked copies are held.
template <typename T>
__device__ __forceinline__ float dot16(const U128 &a, const float (&af)[16 / sizeof(T)],
                                       const U128 &b, float c) {
  if constexpr (__is_same(T, f16)) {
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      asm("v_fma_mix_f32 %0, %1, %2, %0 op_sel_hi:[1,1,0]" : "+v"(c) : "v"(aw[p]), "v"(bw[p]));
      asm("v_fma_mix_f32 %0, %1, %2, %0 op_sel:[1,1,0] op_sel_hi:[1,1,0]" : "+v"(c)
          : "v"(aw[p]), "v"(bw[p]));
    }
  } else {
    const Elems16<T> be = elems16<T>(b);
#pragma unroll
    for (int e = 0; e < 16 / (int)sizeof(T); ++e) c += af[e] * to_f32(be.e[e]);
  }
  return c;
}
template <typename T>
__device__ __forceinline__ void axpy16(float a, const U128 &b, float (&o)[16 / sizeof(T)]) {
  if constexpr (__is_same(T, f16)) {
    const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      asm("v_fma_mix_f32 %0, %1, %2, %0 op_sel_hi:[0,1,0]" : "+v"(o[2 * p]) : "v"(a), "v"(bw[p]));
      asm("v_fma_mix_f32 %0, %1, %2, %0 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "+v"(o[2 * p + 1])
          : "v"(a), "v"(bw[p]));
    }
  } else {
    const Elems16<T> be = elems16<T>(b);
#pragma unroll
    for (int e = 0; e < 16 / (int)sizeof(T); ++e) o[e] += a * to_f32(be.e[e]);
  }
}

// x * y rounded to fp32 and never fused into a following add, so a product
// used by two code paths gives both the same sums.
__device__ __forceinline__ float mul_rounded(float x, float y) {
#pragma clang fp contract(off)
  return x * y;
}

__device__ __forceinline__ uint32_t order_key_pos(float x) {
  const uint32_t u = __float_as_uint(x + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <typename T, int D>
__global__ void __launch_bounds__(256)
h2o_decode_kernel(const T *__restrict__ q, T *__restrict__ K, T *__restrict__ V,
                  const T *__restrict__ k_new, const T *__restrict__ v_new,
                  const int32_t *__restrict__ write_slot,
                  int32_t *__restrict__ slot_pos, float *__restrict__ acc, T *__restrict__ O,
                  int32_t *__restrict__ evict_slot, int rows, int cap, int cur_len, int k_heavy,
                  int k_recent, float c) {
  constexpr int EPC = 16 / (int)sizeof(T);
  constexpr int LPR = D / EPC;  // lanes per slot row
  constexpr int RPI = 64 / LPR; // slot rows per wave step
  constexpr int U = 8;          // wave steps per batch of loads
  constexpr int STEP = RPI * U; // slots per batch
  extern __shared__ float dsh[];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wpb = blockDim.x >> 6;
  const long row = (long)blockIdx.x * wpb + wv;
  if (row >= rows) return;
  float *prob = dsh + (long)wv * 3 * cap;
  float *acc_s = prob + cap;
  int32_t *pos_s = reinterpret_cast<int32_t *>(prob + 2 * cap);
  int32_t *pos = slot_pos + row * cap;
  float *ac = acc + row * cap;
  T *Kr = K + row * cap * D;
  T *Vr = V + row * cap * D;
  const uint32_t row_bytes = (uint32_t)cap * (uint32_t)(D * sizeof(T));
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kr, row_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vr, row_bytes);
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(pos, (uint32_t)cap * 4u);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(ac, (uint32_t)cap * 4u);
  const int newpos = cur_len - 1;
  const int sub = lane % LPR, rr = lane / LPR;

  // the new token's query, key and value, loaded before the slot map
  const U128 qq = *reinterpret_cast<const U128 *>(q + row * D + sub * EPC);
  const U128 kq = *reinterpret_cast<const U128 *>(k_new + row * D + sub * EPC);
  const U128 vq = *reinterpret_cast<const U128 *>(v_new + row * D + sub * EPC);

  // slot map and accumulators into LDS, eight 64-slot blocks per lane loaded
  // together; lowest free slot, how many slots hold a token, and the highest
  // that does
  int ws = -1, nvalid = 0, top = -1;
  for (int base = 0; base < cap; base += 64 * 8) {
    int pv[8];
    float av[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = base + 64 * u + lane;
      const uint32_t off = s < cap ? (uint32_t)s * 4u : kNoLoad;
      pv[u] = __float_as_int(buf_load_f32(rp, off));
      av[u] = buf_load_f32(ra, off);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = base + 64 * u + lane;
      if (s < cap) {
        pos_s[s] = pv[u];
        acc_s[s] = av[u];
      }
      const unsigned long long fb = __ballot(s < cap && pv[u] < 0);
      const unsigned long long vb = __ballot(s < cap && pv[u] >= 0);
      nvalid += __popcll(vb);
      if (ws < 0 && fb) ws = base + 64 * u + __ffsll((long long)fb) - 1;
      if (vb) top = base + 64 * u + 63 - __clzll((long long)vb);
    }
  }
  wave_lds_sync();
  if (write_slot) {
    // the caller's slot: used only if it is in range and free
    const int w = write_slot[row];
    ws = (w >= 0 && w < cap && pos_s[w] < 0) ? w : -1;
  }
  if (ws < 0) {
    if (lane == 0 && evict_slot) evict_slot[row] = -2;
    return;
  }

  // Slots at or above `hi` hold nothing and are not the new token's, so the
  // passes over the slots stop at the batch that covers hi - 1: with the
  // lowest free slot taking each new token and at most one eviction a step,
  // the occupied slots stay a prefix with at most one hole, and a cache that
  // is still filling skips its free tail.  prob[] is written for every slot
  // below hiS and read only there.
  const int hi = max(top, ws) + 1;
  const int hiS = min(cap, (hi + STEP - 1) / STEP * STEP);

  // the query unpacked (unused for fp16, whose FMAs read the packed chunk)
  float qv[EPC];
  {
    const Elems16<T> qe = elems16<T>(qq);
#pragma unroll
    for (int e = 0; e < EPC; ++e) qv[e] = to_f32(qe.e[e]);
  }

  // A batch is U wave steps of slot rows; a slot row is read only if it holds
  // a token other than the one in the new token's slot.
  auto load_batch = [&](U128 *buf, __amdgpu_buffer_rsrc_t r, int base, bool want) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = base + u * RPI + rr;
      const bool ld = want && s < cap && s != ws && pos_s[s] >= 0;
      buf[u] = buf_load16(r, ld ? (uint32_t)(s * D + sub * EPC) * (uint32_t)sizeof(T) : kNoLoad);
    }
  };

  // logits of every valid slot; the new token's slot, whose load is skipped,
  // takes its key from registers.  The row maximum is kept in registers on
  // the way, so the softmax needs no pass of its own for it.
  U128 cur[U];
  float mx = -INFINITY;
  for (int base = 0; base < hiS; base += STEP) {
    load_batch(cur, rk, base, true);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = base + u * RPI + rr;
      const bool inb = s < cap;
      const bool valid = inb && (s == ws || pos_s[s] >= 0);
      float part = dot16<T>(qq, qv, s == ws ? kq : cur[u], 0.f);
      part = lane_group_sum<LPR>(part);
      const float lg = valid ? part * c : -INFINITY;
      mx = fmaxf(mx, lg);
      if (sub == 0 && inb) prob[s] = lg;
    }
  }
  mx = wave_max_dpp(mx);
  wave_lds_sync();
  // the first batch of value rows is in flight during the softmax: issued
  // after the LDS fence, and without a branch on O (no output: nothing is
  // read), so no wait for it is placed before the softmax
  load_batch(cur, rv, 0, O != nullptr);

  // one pass forms the exponentials (kept in prob[]) and their sum; the
  // probabilities a = e / l are formed where they are used, in the pass over
  // the value rows and in the accumulator pass (the same code with and
  // without the output, so both leave the same accumulators).  a is a
  // rounded product, never contracted into the accumulator's add, so the
  // value pass and the accumulators use the same a.
  float l = 0.f;
  for (int s = lane; s < hiS; s += 64) {
    const float e = hw_exp2(prob[s] - mx);
    prob[s] = e;
    l += e;
  }
  l = wave_sum_dpp(l);
  const float inv = 1.f / l;
  wave_lds_sync();

  if (O) {
    float ov[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) ov[e] = 0.f;
    for (int base = 0; base < hiS; base += STEP) {
      if (base > 0) load_batch(cur, rv, base, true);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int s = base + u * RPI + rr;
        const float a = s < hiS ? mul_rounded(prob[s], inv) : 0.f;
        axpy16<T>(a, s == ws ? vq : cur[u], ov);
      }
    }
#pragma unroll
    for (int e = 0; e < EPC; ++e) ov[e] = across_groups_sum<LPR>(ov[e]);
    if (rr == 0) {
      Elems16<T> oe;
#pragma unroll
      for (int e = 0; e < EPC; ++e) oe.e[e] = from_f32<T>(ov[e]);
      *reinterpret_cast<U128 *>(O + row * D + sub * EPC) = pack16(oe);
    }
  }

  // the new token takes its slot
  if (rr == 0) {
    *reinterpret_cast<U128 *>(Kr + (long)ws * D + sub * EPC) = kq;
    *reinterpret_cast<U128 *>(Vr + (long)ws * D + sub * EPC) = vq;
  }
  if (lane == 0) pos[ws] = newpos;

  // One pass adds each retained token's probability to its accumulator and,
  // when the cache is over budget, finds the eviction candidate: the lowest
  // accumulator outside the recent window, the later position on ties.
  // Every occupied slot and the new token's lie below hiS.
  const bool over = nvalid + 1 > k_heavy + k_recent;
  const int recent_from = cur_len - k_recent;
  unsigned long long best = ~0ull;
  for (int s = lane; s < hiS; s += 64) {
    const int p = (s == ws) ? newpos : pos_s[s];
    if (p < 0) continue;
    const float na = ((s == ws) ? 0.f : acc_s[s]) + mul_rounded(prob[s], inv);
    ac[s] = na;
    if (over && p < recent_from) {
      const unsigned long long key =
          ((unsigned long long)order_key_pos(na) << 32) | (uint32_t)(0x7FFFFFFF - p);
      best = key < best ? key : best;
    }
  }
  int ev = -1;
  if (over) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const unsigned long long other = __shfl_xor(best, o, 64);
      best = other < best ? other : best;
    }
    if (best != ~0ull) {
      const int pev = 0x7FFFFFFF - (int)(uint32_t)(best & 0xFFFFFFFFull);
      int cand = -1;
      for (int s = lane; s < hiS; s += 64) {
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

// Waves (rows) per workgroup: four while their probabilities, accumulators
// and slot maps fit 64 KB of LDS, else two (up to 2730 slots).
static inline int decode_waves_per_block(int cap) { return 3 * 4 * cap * 4 <= 65536 ? 4 : 2; }

template <typename T, int D>
static hipError_t run_decode(int rows, int cap, int cur_len, int k_heavy, int k_recent,
                             const void *q, void *K, void *V, const void *k_new,
                             const void *v_new, const int32_t *write_slot, int32_t *slot_pos,
                             float *acc, void *O, int32_t *evict_slot, hipStream_t st) {
  const float c = kLog2e / sqrtf((float)D);
  const int wpb = decode_waves_per_block(cap);
  // probabilities, accumulators and slot map per wave
  const size_t shm = sizeof(float) * 3 * (size_t)cap * wpb;
  {
    TimedLaunch tl_("h2o_decode", st);
    hipLaunchKernelGGL((h2o_decode_kernel<T, D>), dim3((rows + wpb - 1) / wpb), dim3(64 * wpb), shm, st,
                       (const T *)q, (T *)K, (T *)V, (const T *)k_new, (const T *)v_new, write_slot,
                       slot_pos, acc, (T *)O, evict_slot, rows, cap, cur_len, k_heavy, k_recent, c);
  }
  return hipGetLastError();
}

hipError_t launch_h2o_decode(int etype, int d, int rows, int cap, int cur_len, int k_heavy,
                             int k_recent, const void *q, void *K, void *V, const void *k_new,
                             const void *v_new, const int32_t *write_slot, int32_t *slot_pos,
                             float *acc, void *O, int32_t *evict_slot, hipStream_t st) {
#define KVS_D(T, DD)                                                                          \
  return run_decode<T, DD>(rows, cap, cur_len, k_heavy, k_recent, q, K, V, k_new, v_new,     \
                           write_slot, slot_pos, acc, O, evict_slot, st)
  if (etype == E_F32) { if (d == 64) KVS_D(float, 64); KVS_D(float, 128); }
  if (etype == E_BF16) { if (d == 64) KVS_D(bf16, 64); KVS_D(bf16, 128); }
  if (d == 64) KVS_D(f16, 64);
  KVS_D(f16, 128);
#undef KVS_D
}

}  // namespace kvs
