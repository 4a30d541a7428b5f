// Merge of the chunk partials of each (b, h) row.
//
// Without recomputed chunks every partial was taken against the same constant
// phi, so the merge is a plain sum: out = sum_c o_c / sum_c l_c, no rescale
// (FlashDecoding++ theory page, section 3: after the unified maximum only a
// simple sum is left at the end).  A row with a recomputed chunk holds
// partials against different maxima (phi, or the chunk's own maximum) and is
// merged with the ordinary max rescale of split-KV softmax (the split-KV
// figure of section 1).
//
// Two placements.  A grid of at most one round of workgroups (a latency-bound
// call) merges inside the chunk kernel: the last workgroup to finish a row
// group merges it, and the call is one launch.  Larger grids merge in a
// separate launch: there, the per-unit publication below (store completion
// plus a device-scope atomic, under a saturated read stream) costs more than
// the second launch (measured 1-33% slower on the large workloads).
//
// "Last" is decided by a counter per row group in the workspace.  Counters
// are 64-bit words: the high half holds the epoch of the call that wrote it,
// the low half a count.  Every call brings a new epoch, so a word left by an
// earlier call (or never written) is re-based to this call's epoch by the
// first workgroup that touches it -- the workspace needs no initialisation
// -- and the last workgroup resets its row group's count to zero, so a
// launch replayed with the same epoch also starts from zero.
//
// Visibility across the chip's L2 caches: partials are written and read with
// device-coherent (agent-scope) accesses, which bypass the non-coherent cache
// levels, and a workgroup waits for its partial stores to complete before it
// bumps the counter.  The ordinary acquire/release fences would instead write
// back and invalidate a whole L2 at every unit -- measured at 4-5x the time of
// the call.
#pragma once

#include "fd_common.h"

namespace fd {

// Adds `add` to an epoch-tagged counter and returns the count after the add.
// The add is one fetch-and-add; it counts if the word it returns carries this
// call's epoch (once a word has it, it keeps it for the rest of the call).
// An add that returns an older epoch landed on a word left by an earlier call
// and is void: the word is re-based to this call's epoch by a
// compare-and-swap, whose winner's add is the first of the call, and the
// losers add again once the word carries the epoch.  Every add made before
// the re-base is overwritten by it, and none can follow it, so each counted
// add is counted once.  (The earlier form read the word before every add: two
// round trips on the unit that completes a row group, whose merge then waits
// for them.)  A call that completes a counter leaves it at zero tagged with
// the next epoch the host will hand out (next_tag), so that on the next call
// on this workspace -- the usual case -- every add counts at once.
//
// epoch_settle() is the part after the fetch-and-add, given the word it
// returned (so that a caller can issue the add early and use it later).
FD_DEV uint32_t epoch_settle(unsigned long long *w, uint32_t epoch, uint32_t add, unsigned long long v)
{
    if ((uint32_t)(v >> 32) == epoch) return (uint32_t)v + add;
    v += add;                                      // the word as this void add left it
    for (;;) {
        if ((uint32_t)(v >> 32) == epoch)
            return (uint32_t)__hip_atomic_fetch_add(w, (unsigned long long)add, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT) + add;
        if (__hip_atomic_compare_exchange_strong(w, &v, ((unsigned long long)epoch << 32) | add,
                                                 __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            return add;
    }
}

FD_DEV unsigned long long fetch_add64(unsigned long long *w, uint32_t add)
{
    return __hip_atomic_fetch_add(w, (unsigned long long)add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

FD_DEV uint32_t epoch_add(unsigned long long *w, uint32_t epoch, uint32_t add)
{
    return epoch_settle(w, epoch, add, fetch_add64(w, add));
}

// A zero count tagged with the epoch the host hands out after `epoch` (it
// counts up and skips 0).  Any other call finds it stale and re-bases it.
FD_DEV unsigned long long next_tag(uint32_t epoch)
{
    const uint32_t e = epoch + 1 == 0 ? 1u : epoch + 1;
    return (unsigned long long)e << 32;
}

// Device-coherent stores and loads of partials.
template <typename T>
FD_DEV void put(T *ptr, T v)
{
    __hip_atomic_store(ptr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T>
FD_DEV T get(const T *ptr)
{
    return __hip_atomic_load(const_cast<T *>(ptr), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Two consecutive floats in one 8-byte device-coherent load.
FD_DEV f32x2 get2(const float *ptr)
{
    const unsigned long long u = __hip_atomic_load(reinterpret_cast<unsigned long long *>(const_cast<float *>(ptr)),
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return f32x2{__uint_as_float((uint32_t)u), __uint_as_float((uint32_t)(u >> 32))};
}

// Partial stores: device-coherent when the chunk kernel merges (another
// workgroup reads them during the launch), otherwise non-temporal (the merge
// launch reads them after this one; with the K/V stream also non-temporal
// this measured +3% on the 32K GQA workload).
template <typename T>
FD_DEV void part_store(const Params &p, T *ptr, T v)
{
    if (p.fused) put(ptr, v);
    else __builtin_nontemporal_store(v, ptr);
}

// First thing of a call, in one thread of the chunk launch.  With a separate
// merge launch -- the only one that adds to the call's recomputed-pair count,
// and it starts after this launch has ended -- the count word is reset here,
// so a launch replayed with the same epoch (a captured graph) also counts
// from zero.  A fused call publishes its count at its end instead
// (merge_group).
FD_DEV void begin_call(const Params &p)
{
    if (!p.fused) put(p.count_word, (unsigned long long)p.epoch << 32);
}

// Chunks a row group's sequence is cut into; an empty sequence still has one
// (empty) unit, so its rows get written.
FD_DEV int units_of(const Params &p, int L)
{
    return L > 0 ? (L + p.chunk - 1) / p.chunk : 1;
}

// Where the partials of one row group (query heads h0 .. h0 + GB - 1 of a
// sequence) live: partial j of head h0 + i is workspace slot
// base + j * stride + i, for j < n.  Fixed chunks: j is the chunk, the
// partials of one chunk are contiguous over all heads of the sequence
// (part_slot).  Balanced shares: j is the share's index among the row
// group's shares, packed GB slots each.
struct Parts {
    size_t base;
    int stride, n;
};

FD_DEV Parts chunk_parts(const Params &p, int b, int h0, int L)
{
    return Parts{part_slot(p, b, h0, 0), p.hq, units_of(p, L)};
}

// The calling workgroup has stored its partials of one unit of row group
// `rg` (whose sequence is cut into `nunits` units).  Publishes them and
// returns, in every thread, whether this workgroup was the last of its row
// group.  `flag` is a workgroup-shared int.  Contains barriers: every thread
// of the workgroup must call it, after storing its partials with part_store().
// Without a fused merge it returns false at once.
FD_DEV bool publish_unit(const Params &p, int rg, int nunits, int &flag)
{
    if (!p.fused) return false;
    __builtin_amdgcn_s_waitcnt(0);   // this wavefront's partial stores have completed
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t n = epoch_add(p.rg_count + rg, p.epoch, 1);
        flag = n == (uint32_t)nunits;
        // the row group is complete: zero its count for the next call (a
        // replay of this launch with the same epoch re-bases it)
        if (flag) put(p.rg_count + rg, next_tag(p.epoch));
    }
    __syncthreads();
    return flag != 0;
}

// A row group of a fused call is complete (merged, or written directly as a
// one-chunk row group), with `total` recomputed (row, chunk) pairs; in one
// thread.  The pairs go into the call's fused count, then (once that add has
// completed) one into the count of completed row groups; the last row group
// publishes the call's count and zeroes both words for the next call (a
// replay of the launch with the same epoch re-bases them).
FD_DEV void finish_group(const Params &p, int total)
{
    if (total) {
        epoch_add(p.fused_count, p.epoch, (uint32_t)total);
        __builtin_amdgcn_s_waitcnt(0);
    }
    const uint32_t n = epoch_add(p.fused_word, p.epoch, 1);
    if ((int)n == p.ngroups) {
        const unsigned long long c = get(p.fused_count);
        const uint32_t cnt = (uint32_t)(c >> 32) == p.epoch ? (uint32_t)c : 0u;
        put(p.count_word, ((unsigned long long)p.epoch << 32) | cnt);
        put(p.fused_word, next_tag(p.epoch));
        put(p.fused_count, next_tag(p.epoch));
    }
}

// Output element `e` (row * 128 + component): fp32, or bf16 rounded to
// nearest even (NaN stays NaN), as the merge writes it.
FD_DEV uint32_t bf16_bits(float x)
{
    const uint32_t u = __float_as_uint(x);
    return (x != x) ? 0x7fc0u : ((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

FD_DEV void store_out(const Params &p, size_t e, float x)
{
    if (p.out_bf16) static_cast<uint16_t *>(p.out)[e] = (uint16_t)bf16_bits(x);
    else static_cast<float *>(p.out)[e] = x;
}

FD_DEV void store_out4(const Params &p, size_t e, f32x4 x)
{
    if (p.out_bf16)
        *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(p.out) + e) =
            u32x2{bf16_bits(x[0]) | (bf16_bits(x[1]) << 16), bf16_bits(x[2]) | (bf16_bits(x[3]) << 16)};
    else *reinterpret_cast<f32x4 *>(static_cast<float *>(p.out) + e) = x;
}

// One wavefront merges up to R rows (b, h[0..nr-1]) at once: writes
// out[b][h][:] and fallback_flags[b][h] and returns the rows' number of
// recomputed chunks (in every lane).  Lane i holds components 2i and 2i + 1,
// so each 8-byte device-coherent load instruction reads one chunk's whole
// 512-byte partial (a 4-byte load per component, or 16-byte pieces split into
// four such loads, fetch every line several times: these loads bypass the
// L2).  kMergePass chunks of every row are in flight per pass; weight sums,
// maxima and flags sit one chunk per lane (64 chunks at a time), are loaded
// with the first pass, and reach the other lanes as scalars, so rows of up to
// kMergePass chunks cost one memory round trip together when no chunk was
// recomputed.  This runs at the end of the launch (the last unit of each row
// group), where only such round trips are left to wait on.
constexpr int kMergePass = 16;

template <int R>
FD_DEV int merge_rows(const Params &p, int b, const int (&h)[R], int nr, int lane, const Parts &pt, int h0)
{
    constexpr int PC = kMergePass;
    const int L = seq_len_of(p, b);
    const int nch = L > 0 ? pt.n : 0;            // an empty row merges to zeros
    const size_t cs = pt.stride;                 // partial c of a row at its base + c * stride
    size_t base[R];
#pragma unroll
    for (int r = 0; r < R; ++r) base[r] = pt.base + (h[r < nr ? r : 0] - h0);

    // one pass of partials: chunks c0 .. c0 + PC - 1 (clamped to the last
    // chunk: every load stays in the row, the extra ones are not added)
    f32x2 v[R][PC];
    auto load_pass = [&](int c0) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (r >= nr) break;
            const float *op = p.o_part + base[r] * kHeadDim + 2 * lane;
#pragma unroll
            for (int u = 0; u < PC; ++u) v[r][u] = get2(op + (size_t)min(c0 + u, nch - 1) * cs * kHeadDim);
        }
    };
    // chunk c64 + lane of every row: weight sum, maximum, flag
    float lc[R], mc[R];
    int fc[R];
    auto load_lane = [&](int c64) {
        const int c = min(c64 + lane, nch - 1);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (r >= nr) break;
            lc[r] = get(p.l_part + base[r] + c * cs);
            mc[r] = get(p.m_part + base[r] + c * cs);
            fc[r] = get(p.cflag + base[r] + c * cs);
        }
    };
    if (nch > 0) {
        load_pass(0);
        load_lane(0);
    }

    // flagged chunks of each row, and the largest chunk maximum if any
    int nflag[R];
    float M[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (r >= nr) break;
        nflag[r] = __popcll(__ballot(lane < nch && fc[r] != 0));
        M[r] = lane < nch ? mc[r] : -INFINITY;
        for (int c = 64 + lane; c - lane < nch; c += 64) {     // rows of more than 64 chunks
            const bool in = c < nch;
            const int cc = in ? c : nch - 1;
            nflag[r] += __popcll(__ballot(in && get(p.cflag + base[r] + cc * cs) != 0));
            if (in) M[r] = fmaxf(M[r], get(p.m_part + base[r] + cc * cs));
        }
        if (nflag[r]) {
#pragma unroll
            for (int x = 1; x < 64; x <<= 1) M[r] = fmaxf(M[r], __shfl_xor(M[r], x));
        } else {
            M[r] = p.phi;
        }
    }

    // without a recomputed chunk every partial is against phi (weight 1):
    // plain sum; otherwise each is rescaled from its own maximum to M
    f32x2 acc[R];
    float lsum[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        acc[r] = f32x2{0.f, 0.f};
        lsum[r] = 0.f;
    }
    for (int c0 = 0; c0 < nch; c0 += PC) {
        if (c0 > 0) {
            load_pass(c0);
            if (c0 % 64 == 0) load_lane(c0);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (r >= nr) break;
            const float gl = (mc[r] == M[r]) ? 1.f : exp2_hw((mc[r] - M[r]) * kLog2e);
            if (c0 % 64 == 0 && c0 + lane < nch) lsum[r] = fmaf(lc[r], gl, lsum[r]);
            const int o = c0 % 64;
#pragma unroll
            for (int u = 0; u < PC; ++u) {
                if (c0 + u < nch) {
                    const float g = nflag[r] ? __builtin_amdgcn_readlane(__float_as_int(gl), o + u) : 0;
                    acc[r] += nflag[r] ? v[r][u] * __int_as_float(g) : v[r][u];
                }
            }
        }
    }

    int total = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (r >= nr) break;
        total += nflag[r];
        float lacc = lsum[r];
#pragma unroll
        for (int x = 1; x < 64; x <<= 1) lacc += __shfl_xor(lacc, x);
        f32x2 res = {0.f, 0.f};
        if (nch > 0) {
            float vs = 1.f;
            if (p.v_scale) vs = p.v_scale[h[r] / p.group];
            res = acc[r] * (vs / lacc);
        }
        const size_t row = (size_t)b * p.hq + h[r];
        if (p.out_bf16) {
            reinterpret_cast<uint32_t *>(p.out)[row * (kHeadDim / 2) + lane] = bf16_bits(res[0]) | (bf16_bits(res[1]) << 16);
        } else {
            reinterpret_cast<f32x2 *>(p.out)[row * (kHeadDim / 2) + lane] = res;
        }
        if (lane == 0) p.flags[row] = nflag[r] ? 1 : 0;
    }
    return total;
}

// The last workgroup of a row group merges rows (b, h0 .. h0 + nrows - 1),
// its NW wavefronts taking rows round-robin, R at a time, and adds the row
// group's recomputed chunks to the call's count.  `total` is a
// workgroup-shared int.
template <int NW, int R = 2>
FD_DEV void merge_group(const Params &p, int b, int h0, int nrows, int &total, const Parts &pt)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    if (threadIdx.x == 0) total = 0;
    __syncthreads();
    int mine = 0;
    for (int r = wave; r < nrows; r += R * NW) {
        int h[R];
#pragma unroll
        for (int k = 0; k < R; ++k) h[k] = h0 + r + k * NW;
        mine += merge_rows<R>(p, b, h, min(R, (nrows - 1 - r) / NW + 1), lane, pt, h0);
    }
    if (lane == 0 && mine) atomicAdd(&total, mine);
    __syncthreads();
    if (threadIdx.x == 0) finish_group(p, total);
}

// Separate merge launch (large grids): RW wavefronts per row, 256 threads per
// workgroup (256 / (64 RW) rows each).  In a wavefront, lanes 0..31 take one
// chunk and lanes 32..63 the next, 4 components per lane; the wavefronts of a
// row split its chunks and meet in LDS.  Each wavefront loads PP chunk pairs
// per pass with all their loads in flight, the first pass together with the
// chunk flags.  It also adds the recomputed (row, chunk) pairs to the call's
// count.
template <int RW>
__global__ __launch_bounds__(256) void merge_kernel(Params p)
{
    constexpr int ROWS = 4 / RW;
    // chunk pairs per wavefront per pass: rows of fewer than 16 chunks (one
    // wavefront each) take 2, longer rows 4
    constexpr int PP = RW == 1 ? 2 : 4;
    __shared__ f32x4 red_o[4][32];
    __shared__ float red_l[4];
    __shared__ int red_n[4];
    __shared__ float red_m[4];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sub = wave % RW;                       // wavefront inside its row
    const int row = blockIdx.x * ROWS + wave / RW;
    const bool live = row < p.batch * p.hq;
    const int b = live ? row / p.hq : 0, h = live ? row % p.hq : 0;
    const int L = live ? seq_len_of(p, b) : 0;
    const int nch = (L + p.chunk - 1) / p.chunk;
    const size_t base = part_slot(p, b, h, 0);   // chunk c at base + c * hq
    const size_t cs = p.hq;
    const int rw0 = (wave / RW) * RW;                // first wavefront of this row
    const int half = lane >> 5, q4 = lane & 31;
    const float *op = p.o_part + base * kHeadDim + 4 * q4;
    constexpr int STEP = 2 * RW;                     // chunks per pass step of all row waves

    // one pass: chunk c0 + 2 sub + half + STEP u (clamped to the last chunk:
    // every load stays in the row, the extra ones are not added)
    f32x4 v[PP];
    float l[PP], m[PP];
    auto load_pass = [&](int c0) {
#pragma unroll
        for (int u = 0; u < PP; ++u) {
            const int c = min(c0 + 2 * sub + half + STEP * u, nch - 1);
            v[u] = *reinterpret_cast<const f32x4 *>(op + (size_t)c * cs * kHeadDim);
            l[u] = p.l_part[base + c * cs];
            m[u] = p.m_part[base + c * cs];
        }
    };
    if (nch > 0) load_pass(0);

    // flagged chunks of the row, and the largest chunk maximum if any
    int nflag = 0;
    for (int c0 = sub * 64; c0 < nch; c0 += 64 * RW) {
        const int c = c0 + lane;
        nflag += __popcll(__ballot(c < nch && p.cflag[base + c * cs] != 0));
    }
    if (RW > 1) {
        if (lane == 0) red_n[wave] = nflag;
        __syncthreads();
        nflag = 0;
#pragma unroll
        for (int w = 0; w < RW; ++w) nflag += red_n[rw0 + w];
    }
    const bool any = nflag != 0;
    float M = p.phi;
    if (any) {
        M = -INFINITY;
        for (int c = sub * 64 + lane; c < nch; c += 64 * RW) M = fmaxf(M, p.m_part[base + c * cs]);
#pragma unroll
        for (int x = 1; x < 64; x <<= 1) M = fmaxf(M, __shfl_xor(M, x));
    }
    if (RW > 1) {
        if (lane == 0) red_m[wave] = M;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < RW; ++w) M = fmaxf(M, red_m[rw0 + w]);
    }

    // without a recomputed chunk every partial is against phi: plain sum;
    // otherwise each is rescaled from its own maximum to M
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float lacc = 0.f;
    for (int c0 = 0; c0 < nch; c0 += STEP * PP) {
        if (c0 > 0) load_pass(c0);
#pragma unroll
        for (int u = 0; u < PP; ++u) {
            if (c0 + 2 * sub + half + STEP * u < nch) {
                const float g = (m[u] == M) ? 1.f : exp2_hw((m[u] - M) * kLog2e);
                acc += v[u] * g;
                lacc = fmaf(l[u], g, lacc);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += __shfl_xor(acc[i], 32);
    lacc += __shfl_xor(lacc, 32);
    if (RW > 1) {
        if (half == 0) red_o[wave][q4] = acc;
        if (lane == 0) red_l[wave] = lacc;
        __syncthreads();
        if (sub != 0) return;
        acc = f32x4{0.f, 0.f, 0.f, 0.f};
        lacc = 0.f;
#pragma unroll
        for (int w = 0; w < RW; ++w) {
            acc += red_o[rw0 + w][q4];
            lacc += red_l[rw0 + w];
        }
    }
    if (!live) return;

    f32x4 r = {0.f, 0.f, 0.f, 0.f};
    if (nch > 0) {
        float vs = 1.f;
        if (p.v_scale) vs = p.v_scale[h / p.group];
        r = acc * (vs / lacc);
    }
    if (half == 0) store_out4(p, (size_t)row * kHeadDim + 4 * q4, r);
    if (lane == 0) {
        p.flags[row] = any ? 1 : 0;
        if (nflag) epoch_add(p.count_word, p.epoch, (uint32_t)nflag);
    }
}

}  // namespace fd
