// Host construction of the SID prefix trie and its device image.
//
// flashrec 0.1.0, Features > Decoding ("SID constraint"): decoding is restricted to
// valid catalog SIDs by a dense or CSR-sparse trie. Here the CSR form is always
// built; depths below mask_depths additionally carry a 256-bit child mask per node
// (the dense form), which the expand kernel reads with one scalar load.
//
// Numbering (a contract the tests check against an independent construction):
// depth-major, lexicographic. Depth d holds node ids [off_d, off_{d+1}) in ascending
// prefix order, so the children of a node form one contiguous id range, in
// ascending code order, and child_begin[] of all internal nodes is one monotone array.
#include <algorithm>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "tcb_host.h"

namespace {

struct KeyItem {
    uint64_t key;
    int64_t item;
};

// Stable LSD radix sort on the low 8*L bits of the key. Equal keys keep their input
// order, so after sorting, the first entry of each run is its lowest catalog row.
void radix_sort(std::vector<KeyItem> &a, int L) {
    std::vector<KeyItem> tmp(a.size());
    for (int pass = 0; pass < L; ++pass) {
        const int sh = 8 * pass;
        size_t cnt[257] = {0};
        for (const auto &e : a) cnt[((e.key >> sh) & 255) + 1]++;
        for (int i = 0; i < 256; ++i) cnt[i + 1] += cnt[i];
        for (const auto &e : a) tmp[cnt[(e.key >> sh) & 255]++] = e;
        a.swap(tmp);
    }
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

tcb_status tcb_trie_build_impl(const uint8_t *sids, int64_t n_items, int32_t L, int32_t V,
                               int32_t mask_depths, tcb_trie **out) {
    using namespace tcb_host;
    if (!sids || !out) return set_error(TCB_E_ARG, "build_trie: null pointer");
    if (n_items <= 0) return set_error(TCB_E_ARG, "build_trie: n_items must be > 0");
    if (L < 1 || L > TCB_MAX_L) return set_error(TCB_E_RANGE, "build_trie: L must be in 1..8");
    if (V < 2 || V > TCB_MAX_V) return set_error(TCB_E_RANGE, "build_trie: V must be in 2..256");
    if (mask_depths < TCB_MASK_AUTO || mask_depths > L)
        return set_error(TCB_E_ARG, "build_trie: mask_depths must be TCB_MASK_AUTO or in 0..L");
    *out = nullptr;

    std::vector<KeyItem> ki;
    try {
        ki.resize((size_t)n_items);
    } catch (const std::bad_alloc &) {
        return set_error(TCB_E_ARG, "build_trie: out of host memory");
    }
    for (int64_t i = 0; i < n_items; ++i) {
        uint64_t k = 0;
        const uint8_t *s = sids + i * L;
        for (int j = 0; j < L; ++j) {
            if (s[j] >= V)
                return set_error(TCB_E_RANGE, "build_trie: item " + std::to_string(i) +
                                                  " level " + std::to_string(j) + " code " +
                                                  std::to_string(s[j]) + " >= V");
            k = (k << 8) | s[j];
        }
        ki[(size_t)i] = {k, i};
    }
    radix_sort(ki, L);

    tcb_trie *t = new (std::nothrow) tcb_trie();
    if (!t) return set_error(TCB_E_ARG, "build_trie: out of host memory");
    t->L = L;
    t->V = V;
    t->n_items = n_items;

    // distinct SIDs (leaves) and their lowest catalog row
    std::vector<uint64_t> leaf;
    leaf.reserve(ki.size());
    for (size_t i = 0; i < ki.size(); ++i) {
        if (i == 0 || ki[i].key != ki[i - 1].key) {
            leaf.push_back(ki[i].key);
            t->leaf_item.push_back((int32_t)ki[i].item);
        }
    }
    std::vector<KeyItem>().swap(ki);
    t->n_distinct = (int64_t)leaf.size();

    // distinct prefixes per depth, ascending (leaf keys are sorted, so each shifted
    // sequence is non-decreasing and runs can be collapsed in one pass)
    std::vector<std::vector<uint64_t>> P(L + 1);
    P[0].push_back(0);
    for (int d = 1; d <= L; ++d) {
        if (d == L) {
            P[d] = leaf;
            continue;
        }
        const int sh = 8 * (L - d);
        for (uint64_t k : leaf) {
            uint64_t p = k >> sh;
            if (P[d].empty() || P[d].back() != p) P[d].push_back(p);
        }
    }
    std::vector<uint64_t>().swap(leaf);
    t->off.assign(L + 2, 0);
    for (int d = 0; d <= L; ++d) {
        t->nodes_per_depth.push_back((int64_t)P[d].size());
        t->off[d + 1] = t->off[d] + (int64_t)P[d].size();
    }
    if (mask_depths == TCB_MASK_AUTO) {
        // masks on every depth whose table (32 bytes per node, cumulative) fits the budget
        mask_depths = 0;
        while (mask_depths < L && (uint64_t)t->off[mask_depths + 1] * 32u <= (uint64_t)TCB_MASK_AUTO_BYTES)
            ++mask_depths;
    }
    t->mask_depths = mask_depths;
    const int64_t n_nodes = t->off[L + 1];
    const int64_t n_internal = t->off[L];
    if (n_nodes >= (int64_t)0xFFFFFFF0) {
        delete t;
        return set_error(TCB_E_RANGE, "build_trie: more than 2^32 nodes");
    }

    t->child_begin.assign((size_t)n_internal + 1, 0);
    t->child_code.assign((size_t)n_nodes, 0);
    for (int d = 0; d < L; ++d) {
        // parents of consecutive depth-(d+1) prefixes are non-decreasing: two pointers
        size_t i = 0;
        const auto &pd = P[d];
        const auto &pn = P[d + 1];
        for (size_t j = 0; j < pn.size(); ++j) {
            const uint64_t parent = pn[j] >> 8;
            const bool first_child = (j == 0) || ((pn[j - 1] >> 8) != parent);
            if (first_child) {
                while (pd[i] != parent) ++i;
                t->child_begin[(size_t)t->off[d] + i] = (uint32_t)(t->off[d + 1] + (int64_t)j);
            }
            t->child_code[(size_t)(t->off[d + 1] + (int64_t)j)] = (uint8_t)(pn[j] & 255);
        }
    }
    t->child_begin[(size_t)n_internal] = (uint32_t)n_nodes;

    const int64_t n_mask = t->off[mask_depths];
    t->mask.assign((size_t)n_mask * 8, 0);
    for (int64_t n = 0; n < n_mask; ++n) {
        for (uint32_t k = t->child_begin[(size_t)n]; k < t->child_begin[(size_t)n + 1]; ++k) {
            const uint32_t c = t->child_code[k];
            t->mask[(size_t)n * 8 + (c >> 5)] |= 1u << (c & 31);
        }
    }

    // device image: [child_begin][child_code][leaf_item][mask], 256-byte aligned sections
    t->o_child_begin = 0;
    t->o_child_code = align256(t->o_child_begin + t->child_begin.size() * 4);
    t->o_leaf = align256(t->o_child_code + t->child_code.size());
    t->o_mask = align256(t->o_leaf + t->leaf_item.size() * 4);
    t->image_bytes = align256(t->o_mask + t->mask.size() * 4 + 4);
    try {
        t->image.assign(t->image_bytes, 0);
    } catch (const std::bad_alloc &) {
        delete t;
        return set_error(TCB_E_ARG, "build_trie: out of host memory");
    }
    std::memcpy(t->image.data() + t->o_child_begin, t->child_begin.data(), t->child_begin.size() * 4);
    std::memcpy(t->image.data() + t->o_child_code, t->child_code.data(), t->child_code.size());
    std::memcpy(t->image.data() + t->o_leaf, t->leaf_item.data(), t->leaf_item.size() * 4);
    if (!t->mask.empty())
        std::memcpy(t->image.data() + t->o_mask, t->mask.data(), t->mask.size() * 4);
    *out = t;
    return TCB_OK;
}
