// identity.cpp -- the identity part of the C ABI: incremental SHA-256 (the
// semantic identity of weights and configuration), the numerical_policy and
// deployment identities of a (region, case) composition table, and the
// per-call table check.  "IsoExec: Eliminating Trainer-Inference Mismatch in
// SkyRL" (agentlenshq), section "Contract Structure and Enforcement": cases
// and regions, composition, claims, SHA-256 identities.  Host code only.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "../../include/iso.h"
#include "sha256.h"

namespace {

static_assert(sizeof(iso_sha256) == sizeof(iso::Sha256), "iso_sha256 mirrors the hash state");

// A composition with its names normalised (zero after the terminating NUL).
struct Entry {
    char region[32];
    char case_name[32];
    const iso_composition *src;
};

bool copy_name(char dst[32], const char src[32])
{
    size_t n = 0;
    while (n < 32 && src[n] != '\0')
        ++n;
    if (n == 0 || n == 32)
        return false;
    for (size_t i = 0; i < n; ++i)
        if ((unsigned char)src[i] < 0x20 || (unsigned char)src[i] > 0x7e)
            return false;
    memset(dst, 0, 32);
    memcpy(dst, src, n);
    return true;
}

bool name_ok(const char *s)
{
    if (!s)
        return false;
    size_t n = strnlen(s, 32);
    return n > 0 && n < 32;
}

int cmp_entry(const Entry &a, const Entry &b)
{
    int c = memcmp(a.region, b.region, 32);
    return c != 0 ? c : memcmp(a.case_name, b.case_name, 32);
}

void put_u32(iso::Sha256 &h, uint32_t v)
{
    uint8_t b[4] = {(uint8_t)v, (uint8_t)(v >> 8), (uint8_t)(v >> 16), (uint8_t)(v >> 24)};
    h.update(b, 4);
}

// Claims: bits 0..3 only, partitions among them, each claimed count a valid
// split of the policy's leaves.
iso_status check_claims(const iso_composition &c)
{
    if (c.claims == 0 || (c.claims & ~0xFu) != 0)
        return ISO_ERR_CLAIM;
    if (c.partitions == 0 || (c.partitions & (c.partitions - 1)) != 0 || c.partitions > 8)
        return ISO_ERR_CLAIM;
    int k = 0;
    while ((1u << k) != c.partitions)
        ++k;
    if (((c.claims >> k) & 1u) == 0)
        return ISO_ERR_CLAIM;
    for (int b = 0; b < 4; ++b) {
        if (((c.claims >> b) & 1u) == 0)
            continue;
        const uint32_t p = 1u << b;
        if (c.policy.schedule != ISO_SCHED_MFMA16X16X32_KASC ? p != 1 : c.policy.leaf_count % p != 0)
            return ISO_ERR_CLAIM;
    }
    return ISO_OK;
}

iso_status sorted_entries(const iso_composition *table, size_t n, std::vector<Entry> &out)
{
    if (!table && n > 0)
        return ISO_ERR_ARG;
    out.resize(n);
    for (size_t i = 0; i < n; ++i) {
        if (!copy_name(out[i].region, table[i].region) ||
            !copy_name(out[i].case_name, table[i].case_name))
            return ISO_ERR_ARG;
        out[i].src = &table[i];
        iso_status s = iso_contract_validate(&table[i].policy);
        if (s != ISO_OK)
            return s;
        if ((s = check_claims(table[i])) != ISO_OK)
            return s;
    }
    std::sort(out.begin(), out.end(),
              [](const Entry &a, const Entry &b) { return cmp_entry(a, b) < 0; });
    for (size_t i = 1; i < n; ++i)
        if (cmp_entry(out[i - 1], out[i]) == 0)
            return ISO_ERR_ARG;
    return ISO_OK;
}

}  // namespace

extern "C" {

iso_status iso_sha256_init(iso_sha256 *s)
{
    if (!s)
        return ISO_ERR_ARG;
    reinterpret_cast<iso::Sha256 *>(s)->reset();
    return ISO_OK;
}

iso_status iso_sha256_update(iso_sha256 *s, const void *data, size_t n)
{
    if (!s || (!data && n > 0))
        return ISO_ERR_ARG;
    if (n > 0)
        reinterpret_cast<iso::Sha256 *>(s)->update(static_cast<const uint8_t *>(data), n);
    return ISO_OK;
}

iso_status iso_sha256_final(iso_sha256 *s, uint8_t out[32])
{
    if (!s || !out)
        return ISO_ERR_ARG;
    reinterpret_cast<iso::Sha256 *>(s)->finish(out);
    return ISO_OK;
}

iso_status iso_table_digests(const iso_composition *table, size_t n,
                             uint8_t numerical_policy[32], uint8_t deployment[32])
{
    if (!numerical_policy || !deployment || n > 0xFFFFFFFFu)
        return ISO_ERR_ARG;
    std::vector<Entry> e;
    iso_status s = sorted_entries(table, n, e);
    if (s != ISO_OK)
        return s;

    static const char kPolicyTag[] = "iso.numerical_policy.table.v1";
    static_assert(sizeof(kPolicyTag) == 30, "30-byte tag with its NUL");
    iso::Sha256 h;
    h.reset();
    h.update(reinterpret_cast<const uint8_t *>(kPolicyTag), sizeof kPolicyTag);
    put_u32(h, (uint32_t)n);
    for (const Entry &x : e) {
        const iso_contract &c = x.src->policy;
        h.update(reinterpret_cast<const uint8_t *>(x.region), 32);
        h.update(reinterpret_cast<const uint8_t *>(x.case_name), 32);
        const uint32_t f[9] = {c.abi_version, c.in_dtype,    c.accum_dtype,
                               c.leaf_count,  c.leaf_size,   c.tree,
                               c.vocab_chunk, c.schedule,    x.src->claims};
        for (uint32_t v : f)
            put_u32(h, v);
    }
    h.finish(numerical_policy);

    static const char kDeployTag[] = "iso.deployment.v1";
    static_assert(sizeof(kDeployTag) == 18, "18-byte tag with its NUL");
    char version[32];
    memset(version, 0, sizeof version);
    strncpy(version, iso_version(), sizeof version - 1);
    h.reset();
    h.update(reinterpret_cast<const uint8_t *>(kDeployTag), sizeof kDeployTag);
    h.update(reinterpret_cast<const uint8_t *>(version), 32);
    put_u32(h, (uint32_t)n);
    for (const Entry &x : e) {
        h.update(reinterpret_cast<const uint8_t *>(x.region), 32);
        h.update(reinterpret_cast<const uint8_t *>(x.case_name), 32);
        put_u32(h, x.src->partitions);
    }
    h.finish(deployment);
    return ISO_OK;
}

iso_status iso_table_check(const iso_composition *table, size_t n, const char *region,
                           const char *case_name, const iso_contract *c, int partitions)
{
    if (!table || !name_ok(region) || !name_ok(case_name) || !c)
        return ISO_ERR_ARG;
    for (size_t i = 0; i < n; ++i) {
        char r[32], k[32];
        if (!copy_name(r, table[i].region) || !copy_name(k, table[i].case_name))
            return ISO_ERR_ARG;
        if (strcmp(r, region) != 0 || strcmp(k, case_name) != 0)
            continue;
        uint8_t want[32];
        iso_status s = iso_contract_digest(&table[i].policy, want);
        if (s != ISO_OK)
            return s;
        if ((s = iso_contract_check(c, want)) != ISO_OK)
            return s;
        if (partitions < 1 || partitions > 8 || (partitions & (partitions - 1)) != 0)
            return ISO_ERR_CLAIM;
        int b = 0;
        while ((1 << b) != partitions)
            ++b;
        return ((table[i].claims >> b) & 1u) ? ISO_OK : ISO_ERR_CLAIM;
    }
    return ISO_ERR_ARG;
}

}  // extern "C"
