// Lossless exponent coding of bf16 weights (DFloat11-style) for the blocks
// that the tiers keep in bf16.
//
// [DF11] "DFloat11: Nen suy luan GPU khong mat du lieu, giam LLM xuong con
// 70% kich thuoc" (vi.news.hada.io), sections "Du dia nen con lai trong
// exponent cua BFloat16" (only the 8-bit exponent has low entropy),
// "Dinh dang DFloat11" (Huffman-coded exponents in EncodedExponent, sign and
// mantissa verbatim in PackedSignMantissa), "Giai ma dua tren LUT phan cap"
// (height-8 subtrees as 256-entry tables, entries 240..255 as pointers,
// CodeLengths), "Kernel GPU hai giai doan va metadata bo tro" (8 stream bytes
// per thread, 5-bit Gaps, one output position per thread block) and "Giai
// nen theo tung transformer block" (one batched call per block).
//
// Format (per matrix of n weights, one code per matrix):
//  - code lengths: Huffman, merging the two nodes of least (weight, order)
//    with leaves ordered by exponent and internal nodes after them; if that
//    is deeper than 32 bits, the optimal 32-bit-limited code by
//    package-merge.  Canonical codewords by (length, exponent).
//  - EncodedExponent: the codes MSB-first (first bit = bit 7 of byte 0),
//    8 n_seg + 8 bytes with n_seg = ceil(total_bits / 64), zero padded.
//  - PackedSignMantissa: n bytes, sign << 7 | mantissa.
//  - Gaps: per 64-bit segment t, (first code start >= 64 t, or total_bits)
//    - 64 t, in [0, 31], packed 5 bits LSB-first; 4 ceil(5 n_seg / 32) + 4
//    bytes.
//  - block_pos: per decoding block of 256 segments, the number of codes that
//    start before it; n_blocks + 1 entries, the last = n.
//  - tables: root + up to 16 sub-tables of 256 bytes; an entry is an
//    exponent (< 240) or 256 - k for sub-table k, numbered in the order that
//    codes walked in canonical order first need them.
//
// Encoding (three kernels after the histogram): per chunk of 8192 weights
// the total code length, a per-matrix scan of the chunk totals, then each
// chunk assembles its bits in LDS and writes whole words, OR-ing only the
// two words it may share with its neighbours.
//
// Decoding, one workgroup per 256 segments: a thread keeps its 16 stream
// bytes (segment plus the overrun of its last code) in registers, walks the
// codes that start in its segment through a fused root table (exponent and
// length in one 16-bit LDS entry) and the byte sub-tables, in steps unrolled
// at compile time so the exponents stay in registers; a workgroup scan of
// the counts gives each thread's output offset, the exponents go to LDS in
// weight order, and the block's weights are written once, coalesced, each
// 8-weight vector assembled from its sign/mantissa and exponent bytes with
// byte permutes.  The
// page decodes every segment twice (count, then write) to save on-chip
// memory; with 160 KB of LDS per CU one decode and an LDS scatter suffice.
#include "launch.h"

#include <algorithm>
#include <numeric>
#include <queue>
#include <tuple>
#include <vector>

namespace woq {

// ====================================================================
// Host: code construction
// ====================================================================
namespace {

// Huffman depths by repeated merging of the two least (weight, order) nodes.
void huffman_depths(const int64_t* hist, int32_t* len) {
    struct Node { int64_t w; int order; };
    auto greater = [](const Node& a, const Node& b) {
        return std::tie(a.w, a.order) > std::tie(b.w, b.order);
    };
    std::priority_queue<Node, std::vector<Node>, decltype(greater)> pq(greater);
    std::vector<int> parent(256 + 256, -1);
    int used = 0;
    for (int s = 0; s < 256; ++s) {
        len[s] = 0;
        if (hist[s] > 0) { pq.push(Node{hist[s], s}); ++used; }
    }
    if (used == 0) return;
    if (used == 1) { len[pq.top().order] = 1; return; }
    int next = 256;
    while (pq.size() > 1) {
        const Node a = pq.top(); pq.pop();
        const Node b = pq.top(); pq.pop();
        parent[a.order] = next;
        parent[b.order] = next;
        pq.push(Node{a.w + b.w, next});
        ++next;
    }
    for (int s = 0; s < 256; ++s) {
        if (hist[s] <= 0) continue;
        int d = 0;
        for (int v = s; parent[v] >= 0; v = parent[v]) ++d;
        len[s] = d;
    }
}

// Optimal lengths bounded by max_len (package-merge, Larmore and Hirschberg).
// Leaves sorted by (weight, exponent); each level's list merges the leaves
// with the previous level's packages (consecutive pairs), a leaf first on
// equal weight; the first 2 (n - 1) items of the last list are selected and
// a leaf's length is the number of selected items containing it.
void package_merge(const int64_t* hist, int max_len, int32_t* len) {
    std::vector<std::pair<int64_t, int>> leaves;
    for (int s = 0; s < 256; ++s) {
        len[s] = 0;
        if (hist[s] > 0) leaves.push_back({hist[s], s});
    }
    std::sort(leaves.begin(), leaves.end());
    const int n = (int)leaves.size();
    if (n <= 1) {
        if (n == 1) len[leaves[0].second] = 1;
        return;
    }
    struct Item { int64_t w; std::vector<uint16_t> cnt; };
    std::vector<Item> prev;
    for (int level = 0; level < max_len; ++level) {
        std::vector<Item> pk;
        for (size_t i = 0; i + 1 < prev.size(); i += 2) {
            Item it{prev[i].w + prev[i + 1].w, prev[i].cnt};
            for (int k = 0; k < n; ++k) it.cnt[k] += prev[i + 1].cnt[k];
            pk.push_back(std::move(it));
        }
        std::vector<Item> cur;
        size_t i = 0, j = 0;
        while (i < leaves.size() || j < pk.size()) {
            if (j >= pk.size() || (i < leaves.size() && leaves[i].first <= pk[j].w)) {
                Item it{leaves[i].first, std::vector<uint16_t>(n, 0)};
                it.cnt[i] = 1;
                cur.push_back(std::move(it));
                ++i;
            } else {
                cur.push_back(std::move(pk[j]));
                ++j;
            }
        }
        prev = std::move(cur);
    }
    std::vector<int> total(n, 0);
    for (int k = 0; k < 2 * (n - 1); ++k)
        for (int q = 0; q < n; ++q) total[q] += prev[k].cnt[q];
    for (int q = 0; q < n; ++q) len[leaves[q].second] = total[q];
}

}  // namespace

int32_t df11_code_build(const int64_t* hist, uint8_t* code_len, uint32_t* codeword,
                        uint8_t* tables, int32_t* n_tables, int64_t* total_bits) {
    int32_t len[256];
    huffman_depths(hist, len);
    if (*std::max_element(len, len + 256) > kDf11MaxLen) package_merge(hist, kDf11MaxLen, len);
    for (int s = kDf11PtrMin; s < 256; ++s)
        if (len[s] > 0) return WOQ_ERR_VALUE;  // these exponents are table pointers
    // canonical codewords in (length, exponent) order
    std::vector<std::pair<int, int>> order;
    for (int s = 0; s < 256; ++s)
        if (len[s] > 0) order.push_back({len[s], s});
    std::sort(order.begin(), order.end());
    uint32_t cw[256] = {0};
    uint64_t code = 0;
    for (size_t k = 0; k < order.size(); ++k) {
        if (k) code = (code + 1) << (order[k].first - order[k - 1].first);
        cw[order[k].second] = (uint32_t)code;
    }
    // hierarchical tables
    std::vector<uint8_t> tab(256, 0);
    std::vector<bool> is_ptr(256, false);
    int nt = 1;
    for (const auto& o : order) {
        const int L = o.first, s = o.second;
        const uint32_t c = cw[s];
        int t = 0, rem = L;
        while (rem > 8) {
            const int idx = (int)((c >> (rem - 8)) & 0xFFu);
            if (!is_ptr[t * 256 + idx]) {
                if (nt > kDf11MaxSub) return WOQ_ERR_VALUE;
                tab.resize((size_t)(nt + 1) * 256, 0);
                is_ptr.resize((size_t)(nt + 1) * 256, false);
                tab[t * 256 + idx] = (uint8_t)(256 - nt);
                is_ptr[t * 256 + idx] = true;
                ++nt;
            }
            t = 256 - tab[t * 256 + idx];
            rem -= 8;
        }
        const uint32_t low = c & ((1u << rem) - 1u);
        for (uint32_t e = low << (8 - rem); e < ((low + 1) << (8 - rem)); ++e) tab[t * 256 + e] = (uint8_t)s;
    }
    int64_t tot = 0;
    for (int s = 0; s < 256; ++s) {
        code_len[s] = (uint8_t)len[s];
        codeword[s] = cw[s];
        tot += hist[s] * (int64_t)len[s];
    }
    std::copy(tab.begin(), tab.end(), tables);
    *n_tables = nt;
    *total_bits = tot;
    return WOQ_OK;
}

// ====================================================================
// Device
// ====================================================================
namespace {

constexpr int kT = 256;
constexpr int kChunk = kDf11Chunk;          // weights per encoding unit
constexpr int kPerThread = kChunk / kT;     // 32 contiguous weights per thread

__device__ __forceinline__ uint32_t exp_of(uint32_t b) { return (b >> 7) & 0xFFu; }

// 32 contiguous bf16 words of one thread as 16 packed pairs; loads past n
// are not issued and read as zero (callers mask by element index).
__device__ __forceinline__ void load32(const uint16_t* src, int64_t e0, int64_t n, uint32_t (&w)[16]) {
    if (e0 + kPerThread <= n) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint4 v = gload_u4(src + e0 + 8 * k);
            w[4 * k] = v.x; w[4 * k + 1] = v.y; w[4 * k + 2] = v.z; w[4 * k + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int64_t e = e0 + 2 * k;
            const uint32_t lo = e < n ? gload<uint16_t>(src + e) : 0u;
            const uint32_t hi = e + 1 < n ? gload<uint16_t>(src + e + 1) : 0u;
            w[k] = lo | (hi << 16);
        }
    }
}
__device__ __forceinline__ uint32_t half_of(const uint32_t (&w)[16], int j) {
    return (j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xFFFFu);
}

// Exclusive workgroup scan (256 threads) of a 32-bit value; also returns the total.
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t* sh, uint32_t& total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) sh[wid] = x;
    __syncthreads();
    uint32_t base = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < kT / 64; ++w) {
        const uint32_t t = sh[w];
        if (w < wid) base += t;
        total += t;
    }
    __syncthreads();
    return base + x - v;
}

// ---- exponent histogram.  Weights concentrate on a few exponents, so many
//      lanes of a wave add to the same bin: 16 LDS copies, chosen by lane
//      mod 16, with a row stride of 257 words (consecutive copies of a bin
//      fall in different banks), leave at most 4 lanes on one address; the
//      copies are summed per workgroup and added to the matrix's bins.
constexpr int kHistCopies = 16;
__global__ __launch_bounds__(kT) void k_df11_hist(const DfMat* __restrict__ mats,
                                                  const int64_t* __restrict__ ubeg, int nmat,
                                                  uint32_t* __restrict__ hist) {
    __shared__ uint32_t h[kHistCopies * 257];
    const int m = find_unit_owner(ubeg, nmat, (int64_t)blockIdx.x);
    const DfMat d = mats[m];
    for (int i = threadIdx.x; i < kHistCopies * 257; i += kT) h[i] = 0u;
    __syncthreads();
    const int64_t e0 = (int64_t)(blockIdx.x - ubeg[m]) * kChunk + (int64_t)threadIdx.x * kPerThread;
    uint32_t w[16];
    load32(d.src, e0, d.n, w);
    uint32_t* mine = h + (threadIdx.x & (kHistCopies - 1)) * 257;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j)
        if (e0 + j < d.n) atomicAdd(mine + exp_of(half_of(w, j)), 1u);
    __syncthreads();
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < kHistCopies; ++k) c += h[k * 257 + threadIdx.x];
    if (c) atomicAdd(hist + (size_t)m * 256 + threadIdx.x, c);
}

// ---- chunk totals of code length
__global__ __launch_bounds__(kT) void k_df11_count(const DfMat* __restrict__ mats,
                                                   const int64_t* __restrict__ ubeg, int nmat,
                                                   const DfCode* __restrict__ codes,
                                                   uint32_t* __restrict__ chunk_bits) {
    __shared__ uint8_t L[256];
    __shared__ uint32_t sh[kT / 64];
    const int m = find_unit_owner(ubeg, nmat, (int64_t)blockIdx.x);
    const DfMat d = mats[m];
    L[threadIdx.x] = codes[m].len[threadIdx.x];
    __syncthreads();
    const int64_t e0 = (int64_t)(blockIdx.x - ubeg[m]) * kChunk + (int64_t)threadIdx.x * kPerThread;
    uint32_t w[16];
    load32(d.src, e0, d.n, w);
    uint32_t s = 0;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j)
        if (e0 + j < d.n) s += L[exp_of(half_of(w, j))];
    uint32_t total;
    block_scan(s, sh, total);
    if (threadIdx.x == 0) chunk_bits[blockIdx.x] = total;
}

// ---- per-matrix exclusive scan of the chunk totals (one workgroup per matrix)
__global__ __launch_bounds__(kT) void k_df11_scan(const int64_t* __restrict__ ubeg,
                                                  const uint32_t* __restrict__ chunk_bits,
                                                  int64_t* __restrict__ chunk_base) {
    __shared__ uint32_t sh[kT / 64];
    const int m = blockIdx.x;
    const int64_t u0 = ubeg[m], u1 = ubeg[m + 1];
    int64_t run = 0;
    for (int64_t u = u0; u < u1; u += kT) {
        const int64_t i = u + threadIdx.x;
        const uint32_t v = i < u1 ? chunk_bits[i] : 0u;
        uint32_t total;
        const uint32_t ex = block_scan(v, sh, total);
        if (i < u1) chunk_base[i] = run + ex;
        run += total;
    }
}

// ---- zero the stream and gap words (OR targets), batched over matrices
__global__ __launch_bounds__(kT) void k_df11_zero(const DfMat* __restrict__ mats,
                                                  const int64_t* __restrict__ zbeg, int nmat) {
    const int m = find_unit_owner(zbeg, nmat, (int64_t)blockIdx.x);
    const DfMat d = mats[m];
    const int64_t enc_words = d.enc_bytes / 4, words = enc_words + d.gap_bytes / 4;
    const int64_t i0 = (int64_t)(blockIdx.x - zbeg[m]) * (kT * 16) + threadIdx.x;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int64_t i = i0 + (int64_t)kT * k;
        if (i < enc_words) gstore<uint32_t>(reinterpret_cast<uint32_t*>(d.enc) + i, 0u);
        else if (i < words) gstore<uint32_t>(reinterpret_cast<uint32_t*>(d.gaps) + (i - enc_words), 0u);
    }
}

// OR a 5-bit gap into the LSB-first packed Gaps array (fields may straddle words).
__device__ __forceinline__ void or_gap(const DfMat& d, int64_t seg, uint32_t gap) {
    const int64_t bit = 5 * seg;
    const int64_t wi = bit >> 5;
    const uint32_t sb = (uint32_t)(bit & 31);
    uint32_t* gw = reinterpret_cast<uint32_t*>(d.gaps) + wi;
    if (wi < d.gap_bytes / 4) atomicOr(gw, gap << sb);
    if (sb > 27 && wi + 1 < d.gap_bytes / 4) atomicOr(gw + 1, gap >> (32 - sb));
}

// ---- write: sign|mantissa bytes, stream bits, gaps, block positions.
// Positions are chunk-local 32-bit bit offsets from the word that holds the
// chunk's first bit (gbase = B0 rounded down to 32).  Every code is OR-ed
// into a zeroed LDS bit buffer as two words (the second 0 unless the code
// crosses a word), so the per-code work has no branch; the rare events (the
// first code of a 64-bit segment or of a 16384-bit decoding block) are
// collected in per-thread bit masks and written afterwards.
__global__ __launch_bounds__(kT) void k_df11_write(const DfMat* __restrict__ mats,
                                                   const int64_t* __restrict__ ubeg, int nmat,
                                                   const DfCode* __restrict__ codes,
                                                   const int64_t* __restrict__ chunk_base,
                                                   const uint32_t* __restrict__ chunk_bits) {
    __shared__ uint32_t cw[256];
    __shared__ uint8_t L[256];
    __shared__ uint32_t sh[kT / 64];
    __shared__ uint32_t bitbuf[kChunk * kDf11MaxLen / 32 + 2];
    const int m = find_unit_owner(ubeg, nmat, (int64_t)blockIdx.x);
    const DfMat d = mats[m];
    cw[threadIdx.x] = codes[m].code[threadIdx.x];
    L[threadIdx.x] = codes[m].len[threadIdx.x];
    const int64_t B0 = chunk_base[blockIdx.x];
    const uint32_t nbits = chunk_bits[blockIdx.x];
    const uint32_t head = (uint32_t)(B0 & 31);
    const uint32_t nw = (head + nbits + 31) >> 5;
    for (uint32_t i = threadIdx.x; i <= nw; i += kT) bitbuf[i] = 0u;  // + one spill word
    __syncthreads();

    const int64_t e0 = (int64_t)(blockIdx.x - ubeg[m]) * kChunk + (int64_t)threadIdx.x * kPerThread;
    const int nv = (int)std::max<int64_t>(0, std::min<int64_t>(kPerThread, d.n - e0));  // valid weights
    uint32_t w[16];
    load32(d.src, e0, d.n, w);
    // the previous weight decides "first code of a segment / block" for this
    // thread's first code (loaded with the thread's own weights)
    const uint32_t prev_bits = (e0 > 0 && nv > 0) ? (uint32_t)gload<uint16_t>(d.src + e0 - 1) : 0u;
    uint32_t len[kPerThread], code[kPerThread];
    uint32_t s = 0;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
        const uint32_t ex = exp_of(half_of(w, j));
        len[j] = j < nv ? (uint32_t)L[ex] : 0u;
        code[j] = len[j] ? cw[ex] : 0u;
        s += len[j];
    }
    uint32_t dummy;
    const uint32_t off = block_scan(s, sh, dummy);

    // sign | mantissa bytes: high byte & 0x80 | low byte & 0x7F, four at a time
    if (nv > 0) {
        uint32_t sm[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint32_t a = w[2 * k], b = w[2 * k + 1];
            const uint32_t hi = __builtin_amdgcn_perm(b, a, 0x07050301u);  // bytes 1, 3 of a, b
            const uint32_t lo = __builtin_amdgcn_perm(b, a, 0x06040200u);  // bytes 0, 2 of a, b
            sm[k] = (hi & 0x80808080u) | (lo & 0x7F7F7F7Fu);
        }
        if (nv == kPerThread) {
            u32x4 a, c;
            a.x = sm[0]; a.y = sm[1]; a.z = sm[2]; a.w = sm[3];
            c.x = sm[4]; c.y = sm[5]; c.z = sm[6]; c.w = sm[7];
            gstore<u32x4>(d.sm + e0, a);
            gstore<u32x4>(d.sm + e0 + 16, c);
        } else {
#pragma unroll
            for (int j = 0; j < kPerThread; ++j)
                if (j < nv) gstore<uint8_t>(d.sm + e0 + j, (uint8_t)(sm[j >> 2] >> (8 * (j & 3))));
        }
    }

    uint32_t lprev = (e0 > 0 && nv > 0) ? (uint32_t)L[exp_of(prev_bits)] : 0u;
    const int64_t gbase = B0 - head;
    const uint32_t g63 = (uint32_t)(gbase & 63), gblk = (uint32_t)(gbase & 16383);
    uint32_t pos = head + off;  // bit offset of the thread's first code, from gbase
    uint32_t seg_ev = 0, blk_ev = 0, lastlen = 0;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
        lastlen = j == nv - 1 ? len[j] : lastlen;
        const uint32_t wi = pos >> 5, o = pos & 31;
        // the code's bits at o .. o + len - 1 of words wi, wi + 1 (MSB first)
        const uint64_t v = len[j] ? (uint64_t)code[j] << (64 - o - len[j]) : 0u;
        atomicOr(&bitbuf[wi], (uint32_t)(v >> 32));
        atomicOr(&bitbuf[wi + 1], (uint32_t)v);
        const bool fresh = len[j] && ((g63 + pos) & 63) < lprev;
        const bool fblk = len[j] && ((gblk + pos) & 16383) < lprev;
        seg_ev |= (fresh ? 1u : 0u) << j;
        blk_ev |= (fblk ? 1u : 0u) << j;
        lprev = len[j] ? len[j] : lprev;
        pos += len[j];
    }
    if (e0 == 0 && nv > 0) { seg_ev |= 1u; blk_ev |= 1u; }  // the matrix's first code

    // events: gaps (5 bits per segment) and block positions
    if (seg_ev | blk_ev) {
        uint32_t q = head + off;
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            const int64_t start = gbase + q;
            if ((seg_ev >> j) & 1u) {
                const int64_t seg = start >> 6;
                const uint32_t gap = (uint32_t)(start & 63);
                if (seg < d.n_seg && gap) or_gap(d, seg, gap);
            }
            if (((blk_ev >> j) & 1u) && (start >> 14) < d.n_blocks)
                gstore<uint32_t>(d.bpos + (start >> 14), (uint32_t)(e0 + j));
            q += len[j];
        }
    }
    if (e0 <= d.n - 1 && d.n - 1 < e0 + kPerThread) {
        // the matrix's last code: a last segment (and block) in which no code starts
        const int64_t last_start = gbase + pos - lastlen;
        if ((last_start >> 6) < d.n_seg - 1) {
            const int64_t seg = d.n_seg - 1;
            const int64_t gap = d.total_bits - 64 * seg;
            if (gap > 0 && gap < 32) or_gap(d, seg, (uint32_t)gap);
        }
        for (int64_t b = std::max<int64_t>((last_start >> 14) + 1, 0); b <= d.n_blocks; ++b)
            gstore<uint32_t>(d.bpos + b, (uint32_t)d.n);
    }
    __syncthreads();

    // words out: the first and last may be shared with neighbouring chunks
    uint32_t* gwords = reinterpret_cast<uint32_t*>(d.enc) + (B0 >> 5);
    const bool shared_first = head != 0, shared_last = ((head + nbits) & 31) != 0;
    const int64_t room = d.enc_bytes / 4 - (B0 >> 5);  // words left in the stream buffer
    for (uint32_t i = threadIdx.x; i < nw && (int64_t)i < room; i += kT) {
        const uint32_t v = __builtin_bswap32(bitbuf[i]);
        if ((i == 0 && shared_first) || (i == nw - 1 && shared_last)) {
            if (v) atomicOr(gwords + i, v);
        } else {
            gstore<uint32_t>(gwords + i, v);
        }
    }
}

// ---- decode
constexpr int kMaxCodes = 64;                    // codes that can start in one 64-bit segment
constexpr int kBlockMax = kT * kMaxCodes;        // weights one block can hold
constexpr int kOutVecs = kBlockMax / 8 / kT + 1; // 8-weight output vectors per thread (bound)
constexpr int kPre = 3;                           // of them loaded before decoding

// Codes longer than 8 bits (rare): sub-tables on bits 8..15, 16..23, 24..31
// of the window; length 0 for a pattern that is no code of these tables.
__device__ __forceinline__ uint32_t decode_long(uint32_t win, uint32_t ptr, const uint8_t* tabs,
                                                const uint8_t* L, int ntab, uint32_t& len) {
    uint32_t t = 256u - ptr;
    for (int sh8 = 16; sh8 >= 0; sh8 -= 8) {
        if ((int)t >= ntab) break;
        const uint32_t v = tabs[t * 256 + ((win >> sh8) & 0xFFu)];
        if (v < kDf11PtrMin) { len = L[v]; return v; }
        t = 256u - v;
    }
    len = 0;
    return 0;
}

// Code C of a thread's segment (compile-time C: the packed exponents stay in
// registers at static indices).  Every lane runs the step; a lane whose
// position reached its bound (or that met a non-code pattern) commits
// nothing and stops.  The 32-bit window at bit q of hi:lo is
// (hi << q) | ((lo >> 1) >> (63 - q)), exact for every q in 0..63.
template <int C>
__device__ __forceinline__ void decode_step(uint32_t& p, uint32_t& lim, uint64_t hi, uint64_t lo,
                                            const uint16_t* root, const uint8_t* tabs,
                                            const uint8_t* L, int ntab,
                                            uint32_t (&pk)[kMaxCodes / 4], uint32_t& cnt) {
    const bool act = p < lim;
    const uint32_t q = p & 63u;
    const uint32_t win = (uint32_t)(((hi << q) | ((lo >> 1) >> (63u - q))) >> 32);
    const uint32_t e = root[win >> 24];
    uint32_t sym = e & 0xFFu, len = e >> 8;
    if (len == 0 && act) sym = decode_long(win, sym, tabs, L, ntab, len);
    const bool ok = act && len != 0;
    pk[C >> 2] |= (ok ? sym : 0u) << (8 * (C & 3));
    cnt = ok ? (uint32_t)(C + 1) : cnt;
    p = ok ? p + len : p;
    lim = ok ? lim : 0u;
}

template <int C>
__device__ __forceinline__ void decode_steps(uint32_t& p, uint32_t& lim, uint64_t hi, uint64_t lo,
                                             const uint16_t* root, const uint8_t* tabs,
                                             const uint8_t* L, int ntab,
                                             uint32_t (&pk)[kMaxCodes / 4], uint32_t& cnt) {
    if constexpr (C < kMaxCodes) {
        decode_step<C>(p, lim, hi, lo, root, tabs, L, ntab, pk, cnt);
        if constexpr ((C & 3) == 3) {
            if (__ballot(p < lim) == 0) return;  // the whole wave is done
        }
        decode_steps<C + 1>(p, lim, hi, lo, root, tabs, L, ntab, pk, cnt);
    }
}

// 8 bf16 words from 8 sign|mantissa bytes (s0, s1) and 8 exponent bytes
// (x0, x1): high byte = s & 0x80 | e >> 1, low byte = e << 7 & 0x80 | s & 0x7F,
// four lanes of bytes at a time, interleaved by byte permutes.
__device__ __forceinline__ u32x4 join8(uint32_t s0, uint32_t s1, uint32_t x0, uint32_t x1) {
    const uint32_t hb0 = (s0 & 0x80808080u) | ((x0 >> 1) & 0x7F7F7F7Fu);
    const uint32_t lb0 = ((x0 << 7) & 0x80808080u) | (s0 & 0x7F7F7F7Fu);
    const uint32_t hb1 = (s1 & 0x80808080u) | ((x1 >> 1) & 0x7F7F7F7Fu);
    const uint32_t lb1 = ((x1 << 7) & 0x80808080u) | (s1 & 0x7F7F7F7Fu);
    u32x4 w;
    // perm(a, b, sel): byte i of the result = byte sel_i of (a:b), b = bytes 0..3
    w.x = __builtin_amdgcn_perm(hb0, lb0, 0x05010400u);
    w.y = __builtin_amdgcn_perm(hb0, lb0, 0x07030602u);
    w.z = __builtin_amdgcn_perm(hb1, lb1, 0x05010400u);
    w.w = __builtin_amdgcn_perm(hb1, lb1, 0x07030602u);
    return w;
}

// Seven waves per SIMD (the LDS limit at about 21 KB per workgroup): the
// register cap of 72 costs a few spills of the prefetched vectors and still
// measured faster than 5 waves without spills or 7 without the prefetch.
__global__ __launch_bounds__(kT, 7) void k_df11_decode(const DfMat* __restrict__ mats,
                                                    const int64_t* __restrict__ ubeg, int nmat) {
    __shared__ uint8_t tabs[(kDf11MaxSub + 1) * 256];
    __shared__ uint16_t root[256];
    __shared__ uint8_t L[256];
    // exponents of the block's weights; weight i sits at i - (g0 & ~7), so
    // every 8-weight output vector is one aligned 8-byte LDS read
    __shared__ __attribute__((aligned(16))) uint8_t outb[kBlockMax + 16];
    __shared__ uint32_t sh[kT / 64];

    const int m = find_unit_owner(ubeg, nmat, (int64_t)blockIdx.x);
    const DfMat d = mats[m];
    const int64_t lb = blockIdx.x - ubeg[m];
    const int tid = threadIdx.x;
    const int ntab = d.n_tables;

    // ---- every global load first: block range, this thread's sign|mantissa
    //      vectors, its 16 stream bytes and gap, the tables
    const int64_t g0 = gload<uint32_t>(d.bpos + lb);
    int64_t g1 = gload<uint32_t>(d.bpos + lb + 1);
    g1 = g1 > d.n ? d.n : g1;
    g1 = g1 < g0 ? g0 : g1;
    const int64_t base = g0 & ~int64_t(7);
    const int64_t nvec = (g1 - base + 7) >> 3;
    f32x2 smv[kPre];
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
        const int64_t v = tid + (int64_t)kT * k;
        const int64_t i0 = base + 8 * v;
        if (v < nvec && i0 >= g0 && i0 + 8 <= g1) smv[k] = gload<f32x2>(d.sm + i0);
    }
    const int64_t seg = lb * kT + tid;
    uint64_t hi = 0, lo = 0;
    uint32_t p = 0, lim = 0;
    if (seg < d.n_seg) {
        const uint8_t* p8 = d.enc + 8 * seg;
        hi = __builtin_bswap64(gload<uint64_t>(p8));
        lo = __builtin_bswap64(gload<uint64_t>(p8 + 8));
        const int64_t gbit = 5 * seg;
        const uint32_t g16 = (uint32_t)gload<uint8_t>(d.gaps + (gbit >> 3)) |
                             ((uint32_t)gload<uint8_t>(d.gaps + (gbit >> 3) + 1) << 8);
        p = (g16 >> (gbit & 7)) & 31u;
        const int64_t rest = d.total_bits - 64 * seg;
        lim = rest < 64 ? (uint32_t)rest : 64u;
    }
    const uint32_t* gt = reinterpret_cast<const uint32_t*>(d.tables);
    uint32_t* lt = reinterpret_cast<uint32_t*>(tabs);
    for (int i = tid; i < ntab * 64; i += kT) lt[i] = gload<uint32_t>(gt + i);
    if (tid < 64) reinterpret_cast<uint32_t*>(L)[tid] = gload<uint32_t>(reinterpret_cast<const uint32_t*>(d.lens) + tid);
    __syncthreads();
    // fused root: exponent | length << 8 (length 0 marks a pointer)
    {
        const uint32_t v = tabs[tid];
        root[tid] = (uint16_t)(v < kDf11PtrMin ? (v | ((uint32_t)L[v] << 8)) : v);
    }
    __syncthreads();

    // ---- decode the codes that start in this segment, exponents in registers
    uint32_t pk[kMaxCodes / 4];
#pragma unroll
    for (int k = 0; k < kMaxCodes / 4; ++k) pk[k] = 0;
    uint32_t cnt = 0;
    decode_steps<0>(p, lim, hi, lo, root, tabs, L, ntab, pk, cnt);

    // ---- output offsets, exponents into LDS in weight order
    uint32_t total;
    const uint32_t off = block_scan(cnt, sh, total) + (uint32_t)(g0 - base);
#pragma unroll
    for (int c = 0; c < kMaxCodes; ++c) {
        if ((uint32_t)c >= cnt) break;
        outb[off + c] = (uint8_t)(pk[c >> 2] >> (8 * (c & 3)));
    }
    __syncthreads();

    // ---- the block's weights [g0, g0 + count), coalesced
    const int64_t count = std::min<int64_t>(g1 - g0, total);
    if (count <= 0) return;
    const int64_t gend = g0 + count;
#pragma unroll
    for (int k = 0; k < kOutVecs; ++k) {
        const int64_t v = tid + (int64_t)kT * k;
        if (v >= nvec) break;
        const int64_t i0 = base + 8 * v;
        if (i0 >= gend) break;
        if (i0 >= g0 && i0 + 8 <= gend) {
            const uint2 ex = *reinterpret_cast<const uint2*>(outb + 8 * v);
            const f32x2 sv = k < kPre ? smv[k < kPre ? k : 0] : gload<f32x2>(d.sm + i0);
            gstore<u32x4>(d.dst + i0, join8(__float_as_uint(sv.x), __float_as_uint(sv.y), ex.x, ex.y));
        } else {
            for (int64_t i = std::max(i0, g0); i < std::min(i0 + 8, gend); ++i) {
                const uint32_t a = gload<uint8_t>(d.sm + i);
                const uint32_t ea = outb[i - base];
                gstore<uint16_t>(d.dst + i, (uint16_t)(((a & 0x80u) << 8) | (ea << 7) | (a & 0x7Fu)));
            }
        }
    }
}

}  // namespace

hipError_t df11_hist(const DfMat* mats, const int64_t* ubeg, int nmat, int64_t n_units,
                     uint32_t* hist, hipStream_t s) {
    if (n_units <= 0) return hipSuccess;
    k_df11_hist<<<dim3((unsigned)n_units), dim3(kT), 0, s>>>(mats, ubeg, nmat, hist);
    return hipGetLastError();
}

hipError_t df11_encode_run(const DfMat* mats, const int64_t* ubeg, int nmat, int64_t n_units,
                           const int64_t* zbeg, int64_t n_zunits, const DfCode* codes,
                           uint32_t* chunk_bits, int64_t* chunk_base, hipStream_t s) {
    if (n_units <= 0) return hipSuccess;
    k_df11_zero<<<dim3((unsigned)n_zunits), dim3(kT), 0, s>>>(mats, zbeg, nmat);
    k_df11_count<<<dim3((unsigned)n_units), dim3(kT), 0, s>>>(mats, ubeg, nmat, codes, chunk_bits);
    k_df11_scan<<<dim3((unsigned)nmat), dim3(kT), 0, s>>>(ubeg, chunk_bits, chunk_base);
    k_df11_write<<<dim3((unsigned)n_units), dim3(kT), 0, s>>>(mats, ubeg, nmat, codes, chunk_base,
                                                               chunk_bits);
    return hipGetLastError();
}

hipError_t df11_decode_run(const DfMat* mats, const int64_t* ubeg, int nmat, int64_t n_units,
                           hipStream_t s) {
    if (n_units <= 0) return hipSuccess;
    k_df11_decode<<<dim3((unsigned)n_units), dim3(kT), 0, s>>>(mats, ubeg, nmat);
    return hipGetLastError();
}

}  // namespace woq
