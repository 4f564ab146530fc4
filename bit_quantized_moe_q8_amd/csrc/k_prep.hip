// Small per-step kernels of the MoE expert path: q8 activation quantization,
// top-k routing, stable grouping by expert, and the weighted combine.
#include "pq_device.hpp"
#include "pq_internal.hpp"

namespace pqk {

// ---------------------------------------------------------------------------
// q8 activations (Parakon Runtime README, "How it works": int8 activations).
// Eight lanes per 32-value block, four floats per lane (one 16-byte load):
// block max via three xor shuffles, d = max/127, q = round_half_away(x/d).
// ---------------------------------------------------------------------------
// Thread t of a pass quantizes the 4 values 4t..4t+3 (block t/8), already
// loaded in v (zeros past the end); every lane of the 8-lane group takes
// part in the shuffles, in range or not.
__device__ __forceinline__ void q8_lane_v(float4 v, int64_t t, int64_t n_blocks,
                                          int8_t* __restrict__ xq, float* __restrict__ xd) {
    const int64_t blk = t >> 3;
    float d;
    const uint32_t q = q8_pack4(v, d);
    if (blk >= n_blocks) return;
    reinterpret_cast<uint32_t*>(xq)[t] = q;
    if ((t & 7) == 0) xd[blk] = d;
}

__device__ __forceinline__ void q8_lane(const float* __restrict__ x, int64_t t, int64_t n_blocks,
                                        int8_t* __restrict__ xq, float* __restrict__ xd) {
    const float4 v = (t >> 3) < n_blocks ? reinterpret_cast<const float4*>(x)[t] : make_float4(0.f, 0.f, 0.f, 0.f);
    q8_lane_v(v, t, n_blocks, xq, xd);
}

__global__ __launch_bounds__(256) void k_quantize_q8(const float* __restrict__ x,
                                                     int64_t n_blocks,
                                                     int8_t* __restrict__ xq,
                                                     float* __restrict__ xd) {
    q8_lane(x, static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x, n_blocks, xq, xd);
}

hipError_t launch_quantize_q8(const float* x, int64_t n_blocks, int8_t* xq, float* xd,
                              hipStream_t s) {
    if (n_blocks == 0) return hipSuccess;
    const int64_t threads = n_blocks * 8;
    const unsigned grid = static_cast<unsigned>((threads + 255) / 256);
    hipLaunchKernelGGL(k_quantize_q8, dim3(grid), dim3(256), 0, s, x, n_blocks, xq, xd);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Router top-k + softmax over the selected logits (no dropping: llama-modchip
// summary, "Key highlights").  One workgroup per token.  Each logit gets the
// 64-bit key (order-preserving bits of the value, then the complement of its
// expert id), so that a larger key means a larger logit or an equal logit
// with a lower id; the rank of a logit is the number of larger keys, and the
// logits with rank < k are the selection in output order.  One pass, no
// serial arg-max rounds.  -0.0 is folded to +0.0 first (they compare equal).
// ---------------------------------------------------------------------------
constexpr int kRouteMaxExperts = 1024;

__global__ __launch_bounds__(256) void k_route_topk(const float* __restrict__ logits, int T,
                                                    int E, int k, int32_t* __restrict__ ids,
                                                    float* __restrict__ w) {
    __shared__ uint64_t s_key[kRouteMaxExperts];
    __shared__ float s_val[16];
    __shared__ int s_idx[16];
    const int tid = threadIdx.x;
    for (int t = blockIdx.x; t < T; t += gridDim.x) {
        const float* l = logits + static_cast<int64_t>(t) * E;
        for (int e = tid; e < E; e += 256) {
            float v = l[e];
            if (v == 0.0f) v = 0.0f;
            s_key[e] = route_key(v, e);
        }
        __syncthreads();
        for (int e = tid; e < E; e += 256) {
            const uint64_t me = s_key[e];
            int rank = 0;
#pragma unroll 8
            for (int j = 0; j < E; ++j) rank += (s_key[j] > me) ? 1 : 0;
            if (rank < k) {
                s_val[rank] = l[e];
                s_idx[rank] = e;
            }
        }
        __syncthreads();
        if (tid < 64) route_softmax_store(s_val, s_idx, k, tid, ids + static_cast<int64_t>(t) * k,
                                          w + static_cast<int64_t>(t) * k);
        __syncthreads();
    }
}

hipError_t launch_route_topk(const float* logits, int n_tokens, int n_experts, int top_k,
                             int32_t* ids, float* w, hipStream_t s) {
    if (n_tokens == 0) return hipSuccess;
    const int cap = cu_count() * 16;
    const unsigned grid = static_cast<unsigned>(n_tokens < cap ? n_tokens : cap);
    hipLaunchKernelGGL(k_route_topk, dim3(grid), dim3(256), 0, s, logits, n_tokens, n_experts,
                       top_k, ids, w);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Stable grouping by expert (grouped MoE path: pxq_llama README, "What's
// PXQ?").  One workgroup of 8 waves.  Wave w owns the contiguous assignment
// range [w*C, (w+1)*C):
//   1. per-wave histograms hist[w][e] in LDS;
//   2. per expert: exclusive prefix over waves, then an exclusive scan over
//      experts gives expert_offsets, and hist[w][e] becomes the first output
//      slot of wave w's assignments of expert e;
//   3. each wave walks its range 64 at a time in order; lanes with equal keys
//      are found with one ballot per key bit, the rank among them is a
//      popcount of the lower lanes, and the highest lane of each key advances
//      hist[w][e].  Ranks follow assignment order, so the sort is stable.
// ---------------------------------------------------------------------------
constexpr int kGroupWaves = 8;
constexpr int kGroupThreads = kGroupWaves * 64;
constexpr int kGroupMaxExperts = 1024;

__global__ __launch_bounds__(kGroupThreads) void k_group(const int32_t* __restrict__ ids, int A,
                                                         int E, int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ sorted,
                                                         int32_t* __restrict__ active,
                                                         int32_t* __restrict__ n_active) {
    __shared__ int hist[kGroupWaves * kGroupMaxExperts];
    __shared__ int wave_tot[kGroupWaves];
    __shared__ int carry[2];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

    for (int i = tid; i < kGroupWaves * E; i += kGroupThreads) hist[i] = 0;
    __syncthreads();
    const int chunk = (A + kGroupWaves - 1) / kGroupWaves;
    const int beg = min(wave * chunk, A), end = min(beg + chunk, A);
    for (int a = beg + lane; a < end; a += 64) atomicAdd(&hist[wave * E + ids[a]], 1);
    __syncthreads();

    // Experts e = tid + 512*half, processed in two halves to cover E <= 1024.
    int run_off = 0, run_act = 0;
    for (int half = 0; half < 2; ++half) {
        const int e = tid + half * kGroupThreads;
        int cnt = 0;
        if (e < E) {
            for (int w = 0; w < kGroupWaves; ++w) {
                const int h = hist[w * E + e];
                hist[w * E + e] = cnt;
                cnt += h;
            }
        }
        const int off = run_off + block_exclusive_scan(cnt, wave_tot);
        const int act = run_act + block_exclusive_scan(cnt > 0 ? 1 : 0, wave_tot);
        if (e < E) {
            offsets[e] = off;
            for (int w = 0; w < kGroupWaves; ++w) hist[w * E + e] += off;
            if (cnt > 0) active[act] = e;
        }
        if (tid == kGroupThreads - 1) {
            carry[0] = off + cnt;
            carry[1] = act + (cnt > 0 ? 1 : 0);
        }
        __syncthreads();
        run_off = carry[0];
        run_act = carry[1];
        __syncthreads();
    }
    if (tid == 0) {
        offsets[E] = run_off;
        *n_active = run_act;
    }

    int nbits = 1;
    while ((1 << nbits) < E) ++nbits;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base = beg; base < end; base += 64) {
        const int a = base + lane;
        const bool ok = a < end;
        const int key = ok ? ids[a] : 0;
        uint64_t m = __ballot(ok);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = (key >> b) & 1;
            const uint64_t bb = __ballot(ok && bit);
            m &= bit ? bb : ~bb;
        }
        if (ok) {
            const int rank = __popcll(m & below);
            const int pos = hist[wave * E + key] + rank;
            sorted[pos] = a;
            const int leader = 63 - __clzll(m);
            if (leader == lane) hist[wave * E + key] += __popcll(m);
        }
    }
}

hipError_t launch_group(const int32_t* ids, int n_assign, int n_experts, int32_t* offsets,
                        int32_t* sorted, int32_t* active, int32_t* n_active, hipStream_t s) {
    hipLaunchKernelGGL(k_group, dim3(1), dim3(kGroupThreads), 0, s, ids, n_assign, n_experts,
                       offsets, sorted, active, n_active);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fused decode prep for a few tokens: q8 of the activations, top-k routing
// and the stable grouping in one workgroup (one launch instead of three; at
// a handful of tokens each of those is a few microseconds of launch and
// ramp for almost no work).  Results are identical to the three kernels
// above: the same q8 lanes, the same rank-by-key selection and softmax, and
// a grouping that is unique by definition.  Optionally zeroes y (for the
// accumulating combine epilogue of the down mat-vec).
// ---------------------------------------------------------------------------
constexpr int kPrepThreads = 1024;
constexpr int kPrepWaves = kPrepThreads / kWave;
constexpr int kPrepMaxAssign = 256;     // n_tokens * top_k
static_assert(kMaxExperts == kPrepThreads, "one expert per thread in the grouping scans");

__device__ __forceinline__ int prep_block_exclusive_scan(int v, int* wave_tot) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int i = 0; i < wave; ++i) base += wave_tot[i];
    __syncthreads();
    return base + incl - v;
}

__global__ __launch_bounds__(kPrepThreads) void k_decode_prep(
    const float* __restrict__ x, const float* __restrict__ logits, int T, int H, int E, int k,
    int8_t* __restrict__ xq, float* __restrict__ xd, int32_t* __restrict__ ids,
    float* __restrict__ w, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted,
    int32_t* __restrict__ active, int32_t* __restrict__ n_active, float* __restrict__ y_zero) {
    __shared__ uint64_t s_key[kPrepThreads];
    __shared__ float s_val[16][16];
    __shared__ int s_idx[16][16];
    __shared__ int s_ids[kPrepMaxAssign];
    __shared__ int s_tot[kPrepWaves];
    __shared__ int s_carry;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int TE = T * E;
    const bool rank_path = TE <= kPrepThreads;

    // Every load first: this thread's logit (rank path) and its first batch
    // of activations, so the two round trips overlap.
    const float lv = (rank_path && tid < TE) ? logits[tid] : 0.0f;
    const int64_t n_blocks = static_cast<int64_t>(T) * H / 32;
    constexpr int kQ8Batch = 8;
    float4 v[kQ8Batch];
#pragma unroll
    for (int u = 0; u < kQ8Batch; ++u) {
        const int64_t t = u * kPrepThreads + tid;
        v[u] = (t >> 3) < n_blocks ? reinterpret_cast<const float4*>(x)[t] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (rank_path && tid < TE) s_key[tid] = route_key(lv == 0.0f ? 0.0f : lv, tid % E);

    // q8 of x [T][H], eight loads in flight per thread per batch
    for (int64_t base = 0; base < n_blocks * 8; base += kQ8Batch * kPrepThreads) {
        if (base > 0) {
#pragma unroll
            for (int u = 0; u < kQ8Batch; ++u) {
                const int64_t t = base + u * kPrepThreads + tid;
                v[u] = (t >> 3) < n_blocks ? reinterpret_cast<const float4*>(x)[t] : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
#pragma unroll
        for (int u = 0; u < kQ8Batch; ++u) q8_lane_v(v[u], base + u * kPrepThreads + tid, n_blocks, xq, xd);
    }

    // top-k per token over the same 64-bit keys as the separate router (value
    // bits, then the complemented expert id), so the selection and its order
    // are identical.  Up to one key per thread: each thread counts the larger
    // keys of its token (its rank).  More: one wave per token, k rounds of a
    // wave-wide maximum.
    if (rank_path) {
        __syncthreads();
        if (tid < TE) {
            const int t = tid / E;
            const uint64_t me = s_key[tid];
            const uint64_t* row = s_key + t * E;
            int rank = 0;
#pragma unroll 8
            for (int j = 0; j < E; ++j) rank += (row[j] > me) ? 1 : 0;
            if (rank < k) {
                s_val[t][rank] = lv;
                s_idx[t][rank] = tid % E;
            }
        }
    } else {
        for (int t = wave; t < T; t += kPrepWaves) {
            const float* l = logits + static_cast<int64_t>(t) * E;
            uint64_t kk[kMaxExperts / kWave];
#pragma unroll
            for (int i = 0; i < kMaxExperts / kWave; ++i) {
                const int e = lane + kWave * i;
                float lvv = e < E ? l[e] : 0.0f;
                if (lvv == 0.0f) lvv = 0.0f;
                kk[i] = e < E ? route_key(lvv, e) : 0ull;   // real keys are never 0
            }
            for (int r = 0; r < k; ++r) {
                uint64_t mx = 0;
#pragma unroll
                for (int i = 0; i < kMaxExperts / kWave; ++i) mx = kk[i] > mx ? kk[i] : mx;
#pragma unroll
                for (int off = 1; off < kWave; off <<= 1) {
                    const uint64_t o = (static_cast<uint64_t>(static_cast<uint32_t>(__shfl_xor(static_cast<int>(mx >> 32), off))) << 32) |
                                       static_cast<uint32_t>(__shfl_xor(static_cast<int>(mx & 0xffffffffu), off));
                    mx = o > mx ? o : mx;
                }
#pragma unroll
                for (int i = 0; i < kMaxExperts / kWave; ++i)
                    if (kk[i] == mx) kk[i] = 0ull;
                if (lane == 0) {
                    const int e = static_cast<int>(~static_cast<uint32_t>(mx));
                    s_idx[t][r] = e;
                    s_val[t][r] = l[e];
                }
            }
        }
    }
    __syncthreads();
    for (int t = wave; t < T; t += kPrepWaves) {
        route_softmax_store(s_val[t], s_idx[t], k, lane, ids + t * k, w + t * k);
        if (lane < k) s_ids[t * k + lane] = s_idx[t][lane];
    }
    __syncthreads();

    // grouping: thread e counts its expert's assignments (A <= 256), one
    // scan gives the row offset (low 16 bits) and the active-list slot (high
    // 16 bits) together, then thread e lists its assignments in id order
    // (stable)
    const int A = T * k;
    int cnt = 0;
    if (tid < E)
        for (int a = 0; a < A; ++a) cnt += (s_ids[a] == tid) ? 1 : 0;
    const int packed = cnt | ((cnt > 0 ? 1 : 0) << 16);
    const int ex = prep_block_exclusive_scan(packed, s_tot);   // E <= kPrepThreads
    const int off = ex & 0xffff, act = ex >> 16;
    if (tid < E) {
        offsets[tid] = off;
        if (cnt > 0) {
            active[act] = tid;
            int j = off;
            for (int a = 0; a < A; ++a)
                if (s_ids[a] == tid) sorted[j++] = a;
        }
    }
    if (tid == kPrepThreads - 1) s_carry = ex + packed;
    __syncthreads();
    if (tid == 0) {
        offsets[E] = s_carry & 0xffff;
        *n_active = s_carry >> 16;
    }

    if (y_zero) {
        const int64_t n = static_cast<int64_t>(T) * H;
        for (int64_t i = tid; i < n; i += kPrepThreads) y_zero[i] = 0.0f;
    }
}

hipError_t launch_decode_prep(const float* x, const float* logits, int n_tokens, int hidden,
                              int n_experts, int top_k, int8_t* xq, float* xd, int32_t* ids,
                              float* w, int32_t* offsets, int32_t* sorted, int32_t* active,
                              int32_t* n_active, float* y_zero, hipStream_t s) {
    hipLaunchKernelGGL(k_decode_prep, dim3(1), dim3(kPrepThreads), 0, s, x, logits, n_tokens,
                       hidden, n_experts, top_k, xq, xd, ids, w, offsets, sorted, active, n_active,
                       y_zero);
    return hipGetLastError();
}

bool decode_prep_supported(int n_tokens, int n_experts, int top_k) {
    return n_tokens >= 1 && n_tokens <= kPrepWaves && n_experts <= kMaxExperts &&
           n_tokens * top_k <= kPrepMaxAssign && top_k <= 16;
}

// ---------------------------------------------------------------------------
// Load-time validation of a ternary plane: codes equal to 3 (a 2-bit field
// with both bits set) counted over the whole plane by one workgroup.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_validate_ternary(const uint8_t* __restrict__ qs,
                                                           int64_t n_bytes, int32_t* __restrict__ n_bad) {
    __shared__ long long s_part[16];
    const int tid = threadIdx.x;
    long long cnt = 0;
    const int64_t n16 = n_bytes / 16;
    const uint4* q4 = reinterpret_cast<const uint4*>(qs);
    for (int64_t i = tid; i < n16; i += 1024) {
        const uint4 v = q4[i];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) cnt += __popc(w[j] & (w[j] >> 1) & 0x55555555u);
    }
    for (int64_t i = n16 * 16 + tid; i < n_bytes; i += 1024) {
        const uint32_t b = qs[i];
        cnt += __popc(b & (b >> 1) & 0x55u);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off);
    if ((tid & 63) == 0) s_part[tid >> 6] = cnt;
    __syncthreads();
    if (tid == 0) {
        long long tot = 0;
        for (int i = 0; i < 16; ++i) tot += s_part[i];
        *n_bad = tot > 0x7fffffffLL ? 0x7fffffff : static_cast<int32_t>(tot);
    }
}

hipError_t launch_validate_ternary(const uint8_t* qs, int64_t n_bytes, int32_t* n_bad, hipStream_t s) {
    hipLaunchKernelGGL(k_validate_ternary, dim3(1), dim3(1024), 0, s, qs, n_bytes, n_bad);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Weighted combine in slot order: y[t][n] = sum_j w[t][j] * out[t*k+j][n].
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ out,
                                                 const float* __restrict__ w, int T, int k,
                                                 int rows, float* __restrict__ y) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= static_cast<int64_t>(T) * rows) return;
    const int64_t t = i / rows, n = i % rows;
    float acc = 0.0f;
    for (int j = 0; j < k; ++j) acc += w[t * k + j] * out[(t * k + j) * rows + n];
    y[i] = acc;
}

hipError_t launch_combine(const float* out, const float* w, int n_tokens, int top_k, int rows,
                          float* y, hipStream_t s) {
    const int64_t n = static_cast<int64_t>(n_tokens) * rows;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_combine, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
                       out, w, n_tokens, top_k, rows, y);
    return hipGetLastError();
}

}  // namespace pqk
