// The n-gram map drafter (host): prompt lookup generalised ("100 tokens per second ...",
// section "Lever 3: an n-gram overlay for repetition").  The sequence is kept whole; an
// open-addressing table (linear probing, at most half full) holds for every key_len-token
// key the position after its latest occurrence whose continuation exists, with a 32-bit
// hash tag; a match is confirmed against the sequence's own tokens, so there are no false
// hits.
#include <stdint.h>

#include <new>
#include <vector>

#include "vq_internal.h"

struct vq_ngram {
    int32_t k;
    std::vector<int32_t> seq;
    std::vector<int32_t> pos;      // continuation position, -1 = empty slot
    std::vector<uint32_t> tag;
    size_t used = 0;
};

namespace {

// 64-bit hash of the k tokens at t (a multiply-xorshift mix per token).
uint64_t key_hash(const int32_t* t, int k) {
    uint64_t h = 0x9E3779B97F4A7C15ull ^ (uint64_t)k;
    for (int i = 0; i < k; ++i) {
        h ^= (uint64_t)(uint32_t)t[i] + 0x632BE59BD9B4E019ull + (h << 6) + (h >> 2);
        h *= 0xFF51AFD7ED558CCDull;
        h ^= h >> 33;
    }
    h *= 0xC4CEB9FE1A85EC53ull;
    h ^= h >> 29;
    return h;
}

bool same_key(const vq_ngram* m, int32_t p, const int32_t* key) {
    const int32_t* a = m->seq.data() + p - m->k;
    for (int i = 0; i < m->k; ++i)
        if (a[i] != key[i]) return false;
    return true;
}

// Slot of the key at `key` (hash h): its entry, or the empty slot where it would go.
size_t find_slot(const vq_ngram* m, const int32_t* key, uint64_t h) {
    const size_t mask = m->pos.size() - 1;
    const uint32_t tg = (uint32_t)(h >> 32);
    for (size_t i = (size_t)h & mask;; i = (i + 1) & mask) {
        const int32_t p = m->pos[i];
        if (p < 0) return i;
        if (m->tag[i] == tg && same_key(m, p, key)) return i;
    }
}

// Map the key that ends just before position p (which now exists) to p.
void insert(vq_ngram* m, int32_t p) {
    const int32_t* key = m->seq.data() + p - m->k;
    const uint64_t h = key_hash(key, m->k);
    const size_t i = find_slot(m, key, h);
    if (m->pos[i] < 0) {
        m->tag[i] = (uint32_t)(h >> 32);
        ++m->used;
    }
    m->pos[i] = p;
}

void rehash(vq_ngram* m, size_t slots) {
    std::vector<int32_t> old = std::move(m->pos);
    m->pos.assign(slots, -1);
    m->tag.assign(slots, 0u);
    m->used = 0;
    for (int32_t p : old)
        if (p >= 0) insert(m, p);
}

}  // namespace

extern "C" {

int vq_ngram_create(int32_t key_len, vq_ngram** out) {
    vq::clear_error();
    if (!out) return vq::fail(VQ_ERR_ARG, "NULL out");
    *out = nullptr;
    if (key_len < 1 || key_len > 64) return vq::fail(VQ_ERR_ARG, "key_len %d outside 1..64", key_len);
    try {
        vq_ngram* m = new vq_ngram;
        m->k = key_len;
        m->pos.assign(1024, -1);
        m->tag.assign(1024, 0u);
        *out = m;
    } catch (const std::bad_alloc&) {
        return vq::fail(VQ_ERR_HOST, "n-gram map: host allocation failed");
    }
    return VQ_OK;
}

void vq_ngram_destroy(vq_ngram* m) { delete m; }

int vq_ngram_append(vq_ngram* m, const int32_t* tokens, int32_t n) {
    vq::clear_error();
    if (!m) return vq::fail(VQ_ERR_ARG, "NULL map");
    if (n < 0) return vq::fail(VQ_ERR_ARG, "n %d < 0", n);
    if (n == 0) return VQ_OK;
    if (!tokens) return vq::fail(VQ_ERR_ARG, "NULL tokens");
    for (int32_t i = 0; i < n; ++i)
        if (tokens[i] < 0) return vq::fail(VQ_ERR_ARG, "token %d is negative (%d)", i, tokens[i]);
    if ((int64_t)m->seq.size() + n > (int64_t)INT32_MAX) return vq::fail(VQ_ERR_ARG, "sequence past 2^31 - 1 tokens");
    try {
        m->seq.reserve(m->seq.size() + (size_t)n);
        for (int32_t i = 0; i < n; ++i) {
            m->seq.push_back(tokens[i]);
            const int32_t p = (int32_t)m->seq.size() - 1;   // the new token's position
            if (p >= m->k) {
                if (2 * (m->used + 1) > m->pos.size()) rehash(m, 2 * m->pos.size());
                insert(m, p);
            }
        }
    } catch (const std::bad_alloc&) {
        return vq::fail(VQ_ERR_HOST, "n-gram map: host allocation failed");
    }
    return VQ_OK;
}

int vq_ngram_propose(const vq_ngram* m, int32_t max_drafts, int32_t* drafts, int32_t* n_drafts) {
    vq::clear_error();
    if (!m || !n_drafts) return vq::fail(VQ_ERR_ARG, "NULL map or n_drafts");
    if (max_drafts < 0) return vq::fail(VQ_ERR_ARG, "max_drafts %d < 0", max_drafts);
    if (max_drafts > 0 && !drafts) return vq::fail(VQ_ERR_ARG, "NULL drafts");
    *n_drafts = 0;
    const int32_t n = (int32_t)m->seq.size();
    if (max_drafts == 0 || n < m->k) return VQ_OK;
    const int32_t* key = m->seq.data() + n - m->k;
    const size_t i = find_slot(m, key, key_hash(key, m->k));
    const int32_t p = m->pos[i];
    if (p < 0) return VQ_OK;
    const int32_t cnt = max_drafts < n - p ? max_drafts : n - p;
    for (int32_t j = 0; j < cnt; ++j) drafts[j] = m->seq[(size_t)p + j];
    *n_drafts = cnt;
    return VQ_OK;
}

}  // extern "C"
