// Split-count policy and packed-kernel switch resolution of the C ABI.
//
// Follows the "Module attn_splitk" page: parse, parse_gqa_pack,
// resolve_policy, policy_from_env, resolve_gqa_pack, gqa_pack_enabled and
// DECODE_GQA_PACK_DECLARED.  The environment variables keep the names the
// page gives (METRALE_ATTN_DECODE_SPLITK, METRALE_ATTN_DECODE_GQA_PACK) so a
// deployment that sets them gets the same behaviour here.
//
// Readings where the page is silent: whitespace and case folding are ASCII;
// a decimal count is one or more ASCII digits with no sign, and a count too
// large to represent saturates before it is clamped to MAX_DECODE_SPLITS.
#include <ctype.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "pda.h"
#include "pda_geometry.h"

namespace {

// [begin, end) of s with ASCII whitespace removed at both ends.
void trim(const char* s, const char** b, const char** e) {
    const char* p = s;
    const char* q = s + strlen(s);
    while (p < q && isspace((unsigned char)*p)) ++p;
    while (q > p && isspace((unsigned char)q[-1])) --q;
    *b = p;
    *e = q;
}

// Case-insensitive (ASCII) equality of [b, e) with the lower-case word w.
bool word_is(const char* b, const char* e, const char* w) {
    const size_t n = strlen(w);
    if ((size_t)(e - b) != n) return false;
    for (size_t i = 0; i < n; ++i)
        if (tolower((unsigned char)b[i]) != w[i]) return false;
    return true;
}

bool is_off_word(const char* b, const char* e) {
    return word_is(b, e, "0") || word_is(b, e, "off") || word_is(b, e, "false") ||
           word_is(b, e, "no");
}

const char* const kSplitkEnv = "METRALE_ATTN_DECODE_SPLITK";
const char* const kGqaPackEnv = "METRALE_ATTN_DECODE_GQA_PACK";

}  // namespace

extern "C" {

int pda_parse_splitk_policy(const char* s, pda_splitk_policy* out) {
    if (!s || !out) return 0;
    const char *b, *e;
    trim(s, &b, &e);
    if (b == e) return 0;
    if (word_is(b, e, "legacy")) {
        *out = pda_splitk_policy{PDA_SPLITK_LEGACY, 0};
        return 1;
    }
    if (word_is(b, e, "auto")) {
        *out = pda_splitk_policy{PDA_SPLITK_AUTO, 0};
        return 1;
    }
    if (is_off_word(b, e)) {  // split-K off: one split
        *out = pda_splitk_policy{PDA_SPLITK_PINNED, 1};
        return 1;
    }
    uint64_t v = 0;
    for (const char* p = b; p < e; ++p) {
        if (*p < '0' || *p > '9') return 0;
        v = v * 10 + (uint64_t)(*p - '0');
        if (v > 0xFFFFFFFFull) v = 0xFFFFFFFFull;  // saturate; the clamp follows
    }
    *out = pda_splitk_policy{PDA_SPLITK_PINNED, pda_pinned_splits((uint32_t)v)};
    return 1;
}

int pda_parse_gqa_pack(const char* s, int* on) {
    if (!s || !on) return 0;
    const char *b, *e;
    trim(s, &b, &e);
    if (word_is(b, e, "1") || word_is(b, e, "on") || word_is(b, e, "true") ||
        word_is(b, e, "yes")) {
        *on = 1;
        return 1;
    }
    if (is_off_word(b, e)) {
        *on = 0;
        return 1;
    }
    return 0;
}

const char* pda_splitk_declared(void) { return "auto"; }

void pda_resolve_policy(const char* declared, const char* env_value, pda_splitk_policy* out) {
    if (!out) return;
    pda_splitk_policy p{};
    if (env_value && pda_parse_splitk_policy(env_value, &p)) {
        *out = p;
        return;
    }
    if (declared && pda_parse_splitk_policy(declared, &p)) {
        *out = p;
        return;
    }
    *out = pda_splitk_policy{PDA_SPLITK_LEGACY, 0};
}

void pda_policy_from_env(pda_splitk_policy* out) {
    pda_resolve_policy(pda_splitk_declared(), getenv(kSplitkEnv), out);
}

int pda_decode_gqa_pack_declared(void) { return 0; }

int pda_resolve_gqa_pack(int declared, const char* env_value) {
    int on = 0;
    if (env_value && pda_parse_gqa_pack(env_value, &on)) return on;
    return declared ? 1 : 0;
}

int pda_gqa_pack_enabled(void) {
    static std::once_flag once;
    static int enabled = 0;
    std::call_once(once, [] {
        enabled = pda_resolve_gqa_pack(pda_decode_gqa_pack_declared(), getenv(kGqaPackEnv));
    });
    return enabled;
}

}  // extern "C"
