// Block selection into a visible list.
//
// The "attention.rs" page's per-row decode gives row b of a step t_len =
// base_pos + b + 1 positions and blocks = t_len / ratio complete blocks; with
// kblk = budget / ratio a row is selective when blocks > kblk and then attends
// kblk*ratio + (t_len - blocks*ratio) positions (its indexer select pass turns
// block scores into that list; the kernel body is not printed).  Computed
// here: the kblk complete blocks of highest score, ties to the lower block
// index, their positions in ascending order, then the trailing incomplete
// block's positions; with blocks <= kblk that is every position.
//
// MI355X mapping: one 1024-thread workgroup per row.  The row's scores go to
// LDS as order-preserving 32-bit keys (signed zeros merged).  A radix select
// over 4 digits of 8 bits (an LDS histogram per digit, its bins suffix-summed
// by one wave) finds the kblk-th largest key T and how many of the blocks
// equal to T to take.  Two block scans in index order then mark the taken
// ties (the lowest-indexed ones) and give each selected block its slot; all
// threads write the list.  O(blocks) per row whatever the scores.
//
// The optional block bitmask (bit j: the list holds a position of block j)
// comes from the same pass: in the selective case each wave's ballot over its
// 64 blocks of a scan chunk is two mask words (chunks start at multiples of
// 1024 blocks, so words never straddle waves), the trailing block's bit joins
// the ballot of the lane that holds its index, and words past the last chunk
// are written by a final sweep; the dense and tail-only cases have closed
// forms per word.
#include "q8kv_internal.h"
#include "wave_ops.h"

namespace q8kv {
namespace {

constexpr int kSelThreads = 1024;      // a row of up to 1024 blocks in one pass
constexpr int kSelWaves = kSelThreads / kWave;

// Larger key <=> larger score; -0 and +0 map to the same key.
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) == 0) u = 0;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the workgroup of v (0/1 or small counts); also
// returns the total.  tmp: kSelWaves words of LDS.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* tmp, uint32_t& total) {
    const uint32_t lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
    const uint32_t incl = wave_incl_scan(v, lane);
    if (lane == kWave - 1) tmp[wv] = incl;
    __syncthreads();
    uint32_t before = 0;
    total = 0;
#pragma unroll
    for (int i = 0; i < kSelWaves; ++i) {
        const uint32_t t = tmp[i];
        if (static_cast<uint32_t>(i) < wv) before += t;
        total += t;
    }
    __syncthreads();
    return before + incl - v;
}

__global__ __launch_bounds__(kSelThreads) void index_select_kernel(IndexSelectArgs a) {
    __shared__ uint32_t keys[kSelectMaxBlocks];
    __shared__ uint32_t hist[256];
    __shared__ uint32_t tmp[kSelWaves];
    __shared__ uint32_t pick[2];          // digit chosen in this pass, keys still needed after it
    // Indices of the selected blocks, in ascending order.  They share the key
    // array: slot s of block j satisfies s <= j, every key of the current
    // scan chunk is read before the chunk's scans, and later chunks'
    // keys lie above every slot written so far.
    uint32_t* const chosen = keys;
    const uint32_t tid = threadIdx.x, lane = tid % kWave;
    const uint32_t r = blockIdx.x;
    const uint32_t t_len = a.row_lens[r];
    uint32_t blocks = t_len / a.ratio;
    blocks = blocks < a.score_stride ? blocks : a.score_stride;   // out of contract; clamped, not read past the row
    uint32_t* out = a.visible_pos + static_cast<uint64_t>(r) * a.vis_stride;
    const uint32_t k = a.k;
    // head + tail <= vis_stride: the host checks (k + 1)*ratio <= vis_stride, and
    // the tail is shorter than a block unless row_lens breaks its contract.
    const uint32_t head = k * a.ratio;
    uint32_t tail = t_len - blocks * a.ratio;
    tail = tail < a.vis_stride - head ? tail : a.vis_stride - head;
    uint32_t* const bits_out = a.visible_mask ? a.visible_mask + static_cast<uint64_t>(r) * a.mask_stride : nullptr;
    // mask word w when the only touched block (if any) is the trailing one
    const auto tail_word = [&](uint32_t w) -> uint32_t {
        return (tail != 0 && w == blocks / 32) ? 1u << (blocks % 32) : 0u;
    };
    if (blocks > k && k == 0) {                                   // selective, no blocks kept: the tail only
        for (uint32_t e = tid; e < tail; e += kSelThreads) out[e] = blocks * a.ratio + e;
        if (bits_out)
            for (uint32_t w = tid; w < a.mask_stride; w += kSelThreads) bits_out[w] = tail_word(w);
        if (tid == 0) a.num_visible[r] = tail;
        return;
    }
    if (blocks <= k) {                                            // every position
        const uint32_t n = t_len < a.vis_stride ? t_len : a.vis_stride;
        for (uint32_t p = tid; p < n; p += kSelThreads) out[p] = p;
        if (bits_out) {
            const uint32_t nblk = n / a.ratio + (n % a.ratio != 0);   // blocks 0 .. nblk-1 touched
            for (uint32_t w = tid; w < a.mask_stride; w += kSelThreads) {
                const uint32_t lo = w * 32;
                bits_out[w] = nblk >= lo + 32 ? ~0u : (nblk > lo ? (1u << (nblk - lo)) - 1u : 0u);
            }
        }
        if (tid == 0) a.num_visible[r] = n;
        return;
    }
    const float* sc = a.scores + static_cast<uint64_t>(r) * a.score_stride;
    for (uint32_t j = tid; j < blocks; j += kSelThreads) keys[j] = order_key(sc[j]);

    // ---- radix select: T = the k-th largest key, need = how many keys == T to take ----
    uint32_t prefix = 0, mask = 0, need = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
        if (tid < 256) hist[tid] = 0;
        __syncthreads();
        for (uint32_t j = tid; j < blocks; j += kSelThreads) {
            const uint32_t key = keys[j];
            if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid < kWave) {
            // lane l holds digits 255-4l .. 252-4l (descending); suffix sums from the top
            uint32_t h[4], s4 = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) { h[i] = hist[255 - 4 * lane - i]; s4 += h[i]; }
            const uint32_t incl = wave_incl_scan(s4, lane);
            const uint32_t above = incl - s4;                     // keys in higher digits than this lane's
            const uint64_t reach = __ballot(incl >= need);
            const uint32_t l = static_cast<uint32_t>(__builtin_ctzll(reach));
            if (lane == l) {
                uint32_t cum = above, d = 0, left = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (cum + h[i] >= need) { d = 255 - 4 * lane - i; left = need - cum; break; }
                    cum += h[i];
                }
                pick[0] = d;
                pick[1] = left;
            }
        }
        __syncthreads();
        prefix |= pick[0] << shift;
        mask |= 255u << shift;
        need = pick[1];
        __syncthreads();
    }
    const uint32_t T = prefix;

    // ---- index-ordered scans: ties to the lowest indices, then slots ----
    uint32_t eq_run = 0, sel_run = 0;
    for (uint32_t base = 0; base < blocks; base += kSelThreads) {
        const uint32_t j = base + tid;
        const uint32_t key = j < blocks ? keys[j] : 0u;
        const uint32_t eq = (j < blocks && key == T) ? 1u : 0u;
        uint32_t eq_tot, sel_tot;
        const uint32_t eq_before = eq_run + block_excl_scan(eq, tmp, eq_tot);
        const uint32_t sel = (j < blocks && (key > T || (eq && eq_before < need))) ? 1u : 0u;
        const uint32_t slot = sel_run + block_excl_scan(sel, tmp, sel_tot);
        if (sel) chosen[slot] = j;
        if (bits_out) {
            const uint64_t bits = __ballot(sel || (j == blocks && tail != 0));
            const uint32_t w = (j - lane) / 32 + lane;            // this wave's two words; lanes 0 and 1 write
            if (lane < 2 && w < a.mask_stride) bits_out[w] = static_cast<uint32_t>(bits >> (32 * lane));
        }
        eq_run += eq_tot;
        sel_run += sel_tot;
    }
    if (bits_out) {                                               // words past the last scan chunk
        const uint32_t done = (blocks + kSelThreads - 1) / kSelThreads * (kSelThreads / 32);
        for (uint32_t w = done + tid; w < a.mask_stride; w += kSelThreads) bits_out[w] = tail_word(w);
    }
    __syncthreads();

    // ---- the list: k whole blocks ascending, then the tail ----
    for (uint32_t e = tid; e < head; e += kSelThreads) out[e] = chosen[e / a.ratio] * a.ratio + e % a.ratio;
    for (uint32_t e = tid; e < tail; e += kSelThreads) out[head + e] = blocks * a.ratio + e;
    if (tid == 0) a.num_visible[r] = head + tail;
}

}  // namespace

hipError_t launch_index_select(const IndexSelectArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(index_select_kernel, dim3(a.num_rows), dim3(kSelThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace q8kv
