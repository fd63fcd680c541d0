// Ring-attention local step for gfx950: the rank's queries meet every KV
// block, block by block in the order the blocks arrive, folding each into an
// fp32 online-softmax state (m, l, O).
//
// Method: Syncopate summary page, "Experiments" (paper sec. 6.1 and Fig. 9):
// RingAttention among the evaluated operators, with KV blocks passed between
// ranks; the chunk plan makes the kernel wait for each block's ready flag
// before it reads it ("Core method", paper sec. 5).  The per-block merge is the
// usual online softmax: m' = max(m, max s), l' = l e^(m-m') + sum e^(s-m'),
// O' = O e^(m-m') + sum e^(s-m') V.
//
// gfx950 design:
//  * A workgroup (8 wave64s) owns up to 4 query heads that share one KV head
//    (grouped-query attention) and 32 query rows per wave; for 32 query and 8
//    KV heads that is 64 rows x 4 heads, so each K/V tile loaded into LDS is
//    used by 256 query rows.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: a lane then holds 16 keys of one query per
//    32-key block, so the row max and row sum over keys are in-register
//    reductions plus one swap between the two 32-lane halves.
//  * O^T += V^T P^T keeps P in registers: the score accumulator's layout is
//    already the MFMA B-operand layout once the 16 keys of each k-step are
//    taken in the order [0-3, 8-11, 4-7, 12-15].  V stays in LDS as it is in
//    memory (key-major), and gfx950's transposing LDS reads build the V^T
//    fragments, 4 keys per read, in that same key order.  Each lane's O^T
//    column is one query, so the rescale by e^(m-m') is a per-lane multiply.
//  * exp2 with the scale folded into log2(e) units; probabilities go to bf16
//    for the PV product, the running sum stays fp32.
//  * KV tiles of 64 keys, double-buffered in LDS (66 KB), prefetched one tile
//    ahead through registers with 16-byte loads; raw buffer loads return zero
//    past a chunk's last key, and those keys are masked to -inf.
//
// The same kernel runs the head-parallel share (Syncopate summary page,
// "Experiments", paper sec. 6.1 and Fig. 9, head-parallel attention; the
// all-to-all scheme is DeepSpeed-Ulysses', in the review page's references):
// after the all-to-all each rank holds every token of its head group, token
// block w coming from peer w, queries included.  A work item then also waits
// for the chunks holding its own query rows, and items are taken in the
// plan's order (those whose queries land first go first).
#include <math.h>

#include "copy_role.hpp"
#include "device_common.hpp"
#include "launch_args.hpp"

namespace syncov {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kD = 128;           // head dim
constexpr int kKT = 64;           // keys per tile
constexpr int kAttnThreads = 512;  // 8 waves (4 waves in two workgroups per CU measured 13 % slower)
constexpr int kAttnWgPerCu = 512 / kAttnThreads;
constexpr int kKLoads = kKT * 16 / kAttnThreads;  // 16-byte K granules per thread per tile
constexpr int kVLoads = kKT * 16 / kAttnThreads;  // 16-byte V granules per thread per tile
// A work item is HG query heads sharing one KV head (HG = min(heads_q /
// heads_kv, 4)) times 32 * (waves / HG) query rows: one wave per (head, 32 rows).

__device__ __forceinline__ __amdgpu_buffer_rsrc_t attn_rsrc(const void* base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (bytes >= 0x7fffffff ? 0x7fffffff : static_cast<int>(bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), n, 0x00020000);
}

// K rows are padded by one 16-byte slot (16 slots of 8 dims per key), so the
// 16 lanes of a 128-bit read, one row each, start on 16 distinct 4-bank
// groups, and a lane's reads differ from one another by immediate offsets
// only.
constexpr int kKRow = 17;

typedef short s16x4_t __attribute__((ext_vector_type(4)));
// gfx950's transposing LDS read of 16-bit elements: within every group of 16
// lanes, lane i receives element i % 4 of the 8 bytes named by lanes i / 4,
// i / 4 + 4, i / 4 + 8 and i / 4 + 12, in that order.  When lane r of a group
// names row r / 4, columns 4 (r % 4) .. + 3 of a row-major block, lane i
// receives column i, rows 0..3.
__device__ __forceinline__ s16x4_t lds_read_tr16(const void* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(p));
#else
  return s16x4_t{};
#endif
}
// V sits in LDS as it is in memory, [key][16 slots of 8 dims], with 16-byte
// slot s of key k at slot s ^ 4 (k % 4): the 8 keys one transposing read of
// the PV product touches (4 per 32 lanes) then fall on 4 distinct 64-byte
// bank groups, twice.
__device__ __forceinline__ int vswz(int key, int slot) { return slot ^ (4 * (key & 3)); }

// Scheduling hint for a block of N MFMAs fed by N LDS reads: issue AHEAD
// reads first, then alternate one MFMA and one read, so AHEAD reads stay in
// flight instead of one read being waited for before each MFMA.
template <int N, int AHEAD>
__device__ __forceinline__ void sched_reads_ahead() {
  __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);  // LDS reads
#pragma unroll
  for (int i = 0; i < N - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
}


__global__ __launch_bounds__(kAttnThreads, kAttnWgPerCu) void ring_attn_step(AttnArgs a) {
  __shared__ u32x4_t Ks[2][kKT * kKRow];  // [key][16 slots of 8 d + pad]
  __shared__ u32x4_t Vs[2][kKT * 16];     // [key][16 slots of 8 dims, swizzled]
  __shared__ int32_t s_ok;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int HG = a.heads_per_item, QS = (kAttnThreads / 64) / HG, QB = 32 * QS;
  const int hh = wave % HG, qs = wave / HG;
  const int half = lane >> 5, col = lane & 31;
  const uint32_t epoch = call_epoch(a.hdr);
  const int64_t Hq = a.heads_q, Hkv = a.heads_kv;
  const int64_t krow = Hkv * kD;  // elements between consecutive keys of one head
  const float c2 = a.scale * 1.4426950408889634f;  // scale in log2 units
  const int group = static_cast<int>(Hq / Hkv);  // query heads per KV head
  const int nqb = static_cast<int>((a.sq + QB - 1) / QB);
  // per-lane byte offset in a V tile of the first transposing read of dim
  // block b: lane r of 16-lane group g names key 4 (g / 2) + r / 4 and dims
  // 32 b + 16 (g % 2) + 4 (r % 4) .. + 3
  int vrd[4];
  {
    const int g = lane >> 4, r = lane & 15, key = 4 * (g >> 1) + (r >> 2);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int dim = 32 * b + 16 * (g & 1) + 4 * (r & 3);
      vrd[b] = key * 256 + vswz(key, dim >> 3) * 16 + (dim & 7) * 2;
    }
  }
  const int items = a.items ? a.num_items : nqb * static_cast<int>(Hq / HG);

  if (static_cast<int32_t>(blockIdx.x) < a.copy_blocks) {
    copy_role<kAttnThreads>(a.copy, blockIdx.x, a.copy_blocks, epoch);
    end_call(a.hdr, epoch, a.cnt);
    return;
  }
  const int32_t gb = blockIdx.x - a.copy_blocks, gn = gridDim.x - a.copy_blocks;
  if (a.colocated) {  // co-located: pull this workgroup's share of every block first
    if (a.copy.teams > 1)
      copy_role<kAttnThreads>(a.copy, gb, gn, epoch);
    else
      copy_role<kAttnThreads, true>(a.copy, gb, gn, epoch);
  }
  // Chunks this workgroup has already waited for and acquired in this call
  // (ids below 64): later work items read them without another wait, barrier
  // or acquire.  Every thread takes the same waits, so every thread's copy
  // holds the same bits.
  uint64_t known = 0;
  auto is_known = [&](int32_t c) { return c < 64 && ((known >> c) & 1u); };
  auto set_known = [&](int32_t c) {
    if (c < 64) known |= uint64_t(1) << c;
  };
  // head-parallel attention: wait for the chunks holding plan tile t's query rows
  auto wait_queries = [&](int t) {
    if (!a.wait_chunks) return 1;
    bool need = false;
    for (int64_t e = a.dep_ptr[t]; e < a.dep_ptr[t + 1]; ++e) {
      const int32_t c = a.dep_idx[e];
      need = need || !(a.resident[c] || is_known(c));
    }
    if (!need) return 1;
    if (tid == 0) {
      bool ok = true;
      for (int64_t e = a.dep_ptr[t]; ok && e < a.dep_ptr[t + 1]; ++e) {
        const int32_t c = a.dep_idx[e];
        if (!a.resident[c] && !is_known(c)) ok = wait_flag(a.flags, c, epoch, a.hdr, a.timeout_ticks);
      }
      if (ok) acquire_agent();
      s_ok = ok;
    }
    __syncthreads();
    const int ok = s_ok;
    __syncthreads();
    if (ok)
      for (int64_t e = a.dep_ptr[t]; e < a.dep_ptr[t + 1]; ++e) set_known(a.dep_idx[e]);
    return ok;
  };
  const int32_t slot0 = xcd_slot(gb, gn, a.nxcd);
  for (int it = slot0; it < items; it += gn) {
    int hg, qb;
    if (a.items) {  // plan tile t = qb * heads_q + (first head of the group)
      const int t = a.items[it];
      qb = t / static_cast<int>(Hq);
      hg = (t - qb * static_cast<int>(Hq)) / HG;
      if (!wait_queries(t)) continue;  // its queries never arrived: outputs left untouched
    } else {
      hg = it / nqb;  // head-group-major: one KV head's items adjacent
      qb = it - hg * nqb;
    }
    const int64_t h = static_cast<int64_t>(hg) * HG + hh;
    const int g = static_cast<int>(h / group);  // KV head (uniform: HG divides the group or equals it)
    const int64_t q = static_cast<int64_t>(qb) * QB + qs * 32 + col;  // this lane's query row
    const bool qvalid = q < a.sq;

    // Q^T as MFMA B operands: 8 k-steps of 16 dims, 8 dims per lane each.
    bf16x8_t qf[8];
    {
      const __amdgpu_buffer_rsrc_t rq = attn_rsrc(a.q, a.sq * Hq * kD * 2);  // rows past sq read zero
      const uint32_t base = static_cast<uint32_t>(((q * Hq + h) * kD + half * 8) * 2);
#pragma unroll
      for (int ds = 0; ds < 8; ++ds)
        qf[ds] = __builtin_bit_cast(bf16x8_t, __builtin_bit_cast(u32x4_t,
                     __builtin_amdgcn_raw_buffer_load_b128(rq, base + ds * 32, 0, 0)));
    }
    // running state for query q, in log2 units: m2 = max t, l = sum 2^(t - m2)
    float m2, l;
    f32x16_t o[4];
    if (a.init) {
      m2 = -INFINITY;
      l = 0.f;
#pragma unroll
      for (int b = 0; b < 4; ++b) o[b] = f32x16_t{};
    } else {
      m2 = qvalid ? a.m_state[h * a.sq + q] * 1.4426950408889634f : -INFINITY;
      l = qvalid ? a.l_state[h * a.sq + q] : 0.f;
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int dv = b * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
          o[b][i] = qvalid ? a.o[(q * Hq + h) * kD + dv] : 0.f;
        }
    }

    // tile cursor over the chunks in arrival order
    int p = 0;
    int64_t t0 = a.chunk_begin[a.arrival[0]];
    u32x4_t rk[kKLoads], rv[kVLoads];
    auto wait_chunk = [&](int pos) {
      const int32_t c = a.arrival[pos];
      if (!a.wait_chunks || a.resident[c] || is_known(c)) return 1;  // in place, or already acquired
      if (tid == 0) {
        const bool ok = wait_flag(a.flags, c, epoch, a.hdr, a.timeout_ticks);
        if (ok) acquire_agent();
        s_ok = ok;
      }
      __syncthreads();
      const int ok = s_ok;
      __syncthreads();
      if (ok) set_known(c);
      return ok;
    };
    // global -> registers for the tile [t, t + kKT) of chunk at position pos
    auto load_tile = [&](int pos, int64_t t) {
      const int64_t kend = a.chunk_begin[a.arrival[pos] + 1];
      const int64_t bytes = (kend - t - 1) * krow * 2 + kD * 2;  // through the chunk's last key
      const __amdgpu_buffer_rsrc_t rk_ = attn_rsrc(a.k + (t * Hkv + g) * kD, bytes);
      const __amdgpu_buffer_rsrc_t rv_ = attn_rsrc(a.v + (t * Hkv + g) * kD, bytes);
#pragma unroll
      for (int i = 0; i < kKLoads; ++i) {  // K: 64 keys x 16 slots = 1024 granules
        const int gi = tid + i * kAttnThreads, key = gi >> 4, sl = gi & 15;
        rk[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                    rk_, static_cast<uint32_t>((key * krow + sl * 8) * 2), 0, 0));
      }
#pragma unroll
      for (int i = 0; i < kVLoads; ++i) {  // V: the same granules
        const int gi = tid + i * kAttnThreads, key = gi >> 4, sl = gi & 15;
        rv[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                    rv_, static_cast<uint32_t>((key * krow + sl * 8) * 2), 0, 0));
      }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
      for (int i = 0; i < kKLoads; ++i) {
        const int gi = tid + i * kAttnThreads, key = gi >> 4, sl = gi & 15;
        Ks[buf][key * kKRow + sl] = rk[i];
      }
#pragma unroll
      for (int i = 0; i < kVLoads; ++i) {
        const int gi = tid + i * kAttnThreads, key = gi >> 4, sl = gi & 15;
        Vs[buf][key * 16 + vswz(key, sl)] = rv[i];
      }
    };
    auto advance = [&](int& pos, int64_t& t) {  // next tile; pos == C when done
      t += kKT;
      if (t >= a.chunk_begin[a.arrival[pos] + 1]) {
        ++pos;
        if (pos < a.num_chunks) t = a.chunk_begin[a.arrival[pos]];
      }
    };

    bool alive = wait_chunk(0);
    if (alive) {
      load_tile(0, t0);
      store_tile(0);
    }
    __syncthreads();
    int buf = 0;
    while (alive && p < a.num_chunks) {
      const int64_t kend = a.chunk_begin[a.arrival[p] + 1];
      const int valid = static_cast<int>(kend - t0 < kKT ? kend - t0 : kKT);
      int np = p;
      int64_t nt = t0;
      advance(np, nt);
      const bool more = np < a.num_chunks;
      if (more) {
        if (np != p && !wait_chunk(np)) {  // next chunk never arrived
          alive = false;
          break;
        }
        load_tile(np, nt);
      }

      // S^T = K Q^T: two 32-key blocks
      // (the two 32-key blocks' chains alternate; all 16 K fragments are read first)
      f32x16_t s[2] = {f32x16_t{}, f32x16_t{}};
      {
        bf16x8_t kf[8][2];
#pragma unroll
        for (int ds = 0; ds < 8; ++ds)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            kf[ds][kb] = __builtin_bit_cast(bf16x8_t, Ks[buf][(kb * 32 + col) * kKRow + ds * 2 + half]);
#pragma unroll
        for (int ds = 0; ds < 8; ++ds)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ds][kb], qf[ds], s[kb], 0, 0, 0);
        sched_reads_ahead<16, 8>();
      }
      // online softmax for this lane's query over the tile's keys; keys past
      // the chunk's last one (only on its last, partial tile) are masked
      if (valid < kKT) {
        const int lim = valid - 4 * half;  // key - 4 * half is a constant per register
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (kb * 32 + 8 * (i >> 2) + (i & 3) >= lim) s[kb][i] = -INFINITY;
      }
      float mraw = s[0][0];  // tile max of the unscaled scores (scale > 0)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mraw = fmaxf(mraw, s[kb][i]);
      mraw = fmaxf(mraw, __shfl_xor(mraw, 32, 64));
      // (l, O) are rescaled only on tiles where some query's max grows; for
      // the others alpha would be exactly 1, so skipping it changes nothing.
      // The max key of each query keeps probability exactly 1.
      const float mt = mraw * c2;
      if (__ballot(mt > m2)) {
        const float mnew = fmaxf(m2, mt);
        const float alpha = __builtin_amdgcn_exp2f(m2 - mnew);  // 0 on the first tile (m2 = -inf)
        l *= alpha;
#pragma unroll
        for (int b = 0; b < 4; ++b) o[b] *= alpha;
        m2 = mnew;
      }
      const float nm = -m2;
      float lsum = 0.f;
      bf16x8_t pf[4];  // P^T as B operands: k-steps of 16 keys
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(s[kb][i], c2, nm));  // masked keys: exp2(-inf) = 0
          lsum += pv;
          pf[kb * 2 + (i >> 3)][i & 7] = static_cast<__bf16>(pv);
        }
      lsum += __shfl_xor(lsum, 32, 64);
      l += lsum;
      // O^T += V^T P^T: 4 blocks of 32 dims x 4 k-steps of 16 keys.  A
      // fragment's lane holds dim 32 b + lane % 32 at keys 4 h..4 h + 3 and
      // 8 + 4 h..8 + 4 h + 3 of the k-step (h = lane / 32: the order P holds
      // them in), two transposing reads of 4 keys each.
      {
        bf16x8_t vf[4][4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const char* const p = reinterpret_cast<const char*>(Vs[buf]) + ks * 16 * 256 + vrd[b];
            const s16x4_t lo = lds_read_tr16(p), hi = lds_read_tr16(p + 8 * 256);
            vf[ks][b] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int b = 0; b < 4; ++b)
            o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[ks][b], pf[ks], o[b], 0, 0, 0);
        sched_reads_ahead<16, 8>();
      }
      if (more) store_tile(buf ^ 1);
      __syncthreads();
      buf ^= 1;
      p = np;
      t0 = nt;
    }
    if (!alive) continue;  // a block never arrived: this work item's outputs are left untouched

    // write back the state (lanes 0..31 and 32..63 hold the same query)
    if (qvalid) {
      const float ln2 = 0.6931471805599453f;
      if (a.finalize) {
        const float inv = 1.f / l;
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int dv = b * 32 + 8 * i4 + 4 * half;
            float4 v4 = make_float4(o[b][4 * i4] * inv, o[b][4 * i4 + 1] * inv, o[b][4 * i4 + 2] * inv,
                                    o[b][4 * i4 + 3] * inv);
            *reinterpret_cast<float4*>(a.o + (q * Hq + h) * kD + dv) = v4;
          }
        if (half == 0) {
          if (a.lse) a.lse[h * a.sq + q] = m2 * ln2 + logf(l);
          if (a.m_state) {
            a.m_state[h * a.sq + q] = m2 * ln2;
            a.l_state[h * a.sq + q] = l;
          }
        }
      } else {
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int dv = b * 32 + 8 * i4 + 4 * half;
            float4 v4 = make_float4(o[b][4 * i4], o[b][4 * i4 + 1], o[b][4 * i4 + 2], o[b][4 * i4 + 3]);
            *reinterpret_cast<float4*>(a.o + (q * Hq + h) * kD + dv) = v4;
          }
        if (half == 0) {
          a.m_state[h * a.sq + q] = m2 * ln2;
          a.l_state[h * a.sq + q] = l;
        }
      }
    }
  }
  end_call(a.hdr, epoch, a.cnt);
}

hipError_t launch_ring_attn(const AttnArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL(ring_attn_step, dim3(grid), dim3(kAttnThreads), 0, s, a);
  return hipGetLastError();
}

// Workgroups per CU the launch assumes (every one resident: the co-located
// copy publishes once all have copied), and the query rows of a work item
// with hg query heads per item.
int attn_wg_per_cu() { return kAttnWgPerCu; }
int attn_query_block(int hg) { return 32 * ((kAttnThreads / 64) / hg); }

}  // namespace syncov
