/* Seeded random inputs through the CPU oracle's append and decode, for a build
 * of oracle/pa_oracle.c under AddressSanitizer and UndefinedBehaviorSanitizer:
 * every (q, KV) dtype pair, block sizes 16 to 64, ragged and zero lengths,
 * window starts, row subsets, several thread counts, and the refused inputs
 * (a slot or table entry outside the pool, a bad shape).  One value check
 * rides along: a one-token window gives out = v_scale * V of that token. */
#include <stdio.h>

#include "../../oracle/pa_oracle.c"

static uint64_t g_state;
static uint32_t rnd(uint32_t n)
{
    g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(g_state >> 33) % (n ? n : 1);
}

static int g_fail;
static void check(int ok, const char *what, int c)
{
    if (!ok && g_fail < 20) {
        fprintf(stderr, "case %d: %s\n", c, what);
        ++g_fail;
    }
}

/* random bytes of a valid value of the dtype (no NaN codes) */
static void fill(void *p, size_t n, int dt)
{
    for (size_t i = 0; i < n; ++i) {
        if (dt == ORC_F32) {
            ((float *)p)[i] = (float)((int)rnd(2001) - 1000) / 500.0f;
        } else if (dt == ORC_E4M3) {
            uint8_t c = (uint8_t)rnd(256);
            if ((c & 0x7F) == 0x7F)
                c ^= 1;
            ((uint8_t *)p)[i] = c;
        } else {
            /* a small float's 16-bit pattern: sign, exponent near the bias */
            const uint16_t e = dt == ORC_F16 ? (uint16_t)(13 + rnd(4)) : (uint16_t)(125 + rnd(4));
            const int mbits = dt == ORC_F16 ? 10 : 7;
            ((uint16_t *)p)[i] = (uint16_t)((rnd(2) << 15) | (e << mbits) | rnd(1u << mbits));
        }
    }
}

int main(void)
{
    const int pairs[5][2] = {{ORC_F32, ORC_F32}, {ORC_F16, ORC_F16}, {ORC_BF16, ORC_BF16},
                             {ORC_BF16, ORC_E4M3}, {ORC_F16, ORC_E4M3}};
    int c = 0;
    for (int pi = 0; pi < 5; ++pi)
        for (int bsi = 0; bsi < 3; ++bsi)
            for (int rep = 0; rep < 4; ++rep, ++c) {
                g_state = 1000003ull * (uint64_t)c + 17;
                const int qt = pairs[pi][0], kt = pairs[pi][1];
                const int bs = 16 << bsi, D = rep % 2 ? 64 : 128;
                const int Hkv = 1 + (int)rnd(3), G = 1 << rnd(3), Hq = Hkv * G, B = 1 + (int)rnd(5);
                const int qb = orc_elem_bytes(qt), kb = orc_elem_bytes(kt);
                int32_t lens[8], starts[8];
                int maxb = 1;
                for (int b = 0; b < B; ++b) {
                    lens[b] = b == 0 ? 0 : (int32_t)rnd(5 * bs);
                    starts[b] = rnd(3) == 0 ? (int32_t)rnd((uint32_t)lens[b] + 1) : 0;
                    const int nb = (lens[b] + bs - 1) / bs;
                    maxb = nb > maxb ? nb : maxb;
                }
                const int NB = B * maxb + 3;
                int32_t *tables = malloc(sizeof(int32_t) * (size_t)B * maxb);
                int32_t *perm = malloc(sizeof(int32_t) * (size_t)NB);
                for (int i = 0; i < NB; ++i)
                    perm[i] = i;
                for (int i = NB - 1; i > 0; --i) {
                    const int j = (int)rnd((uint32_t)i + 1);
                    const int32_t t = perm[i];
                    perm[i] = perm[j];
                    perm[j] = t;
                }
                int used = 0, ntok = 0;
                for (int b = 0; b < B; ++b)
                    for (int j = 0; j < maxb; ++j)
                        tables[b * maxb + j] = j < (lens[b] + bs - 1) / bs ? perm[used++] : -1;
                for (int b = 0; b < B; ++b)
                    ntok += lens[b];
                /* the append writes every stored token from q-dtype rows */
                const size_t cache_elems = (size_t)NB * Hkv * bs * D;
                void *kc = calloc(cache_elems, (size_t)kb), *vc = calloc(cache_elems, (size_t)kb);
                void *kn = malloc((size_t)(ntok + 1) * Hkv * D * qb);
                void *vn = malloc((size_t)(ntok + 1) * Hkv * D * qb);
                int32_t *slots = malloc(sizeof(int32_t) * (size_t)(ntok + 1));
                fill(kn, (size_t)ntok * Hkv * D, qt);
                fill(vn, (size_t)ntok * Hkv * D, qt);
                int t = 0;
                for (int b = 0; b < B; ++b)
                    for (int p = 0; p < lens[b]; ++p, ++t)
                        slots[t] = rnd(7) == 0 ? -1 : tables[b * maxb + p / bs] * bs + p % bs;
                orc_cache_desc cd = {NB, bs, Hkv, D, kt, qt};
                const float ks = kt == ORC_E4M3 ? 0.01f : 1.0f, vs = kt == ORC_E4M3 ? 0.02f : 1.0f;
                check(orc_cache_append(&cd, kn, vn, kc, vc, slots, ntok, ks, vs) == 0, "append",
                      c);
                /* the skipped slots still hold zeros, so every stored value is finite;
                 * a slot past the pool is refused */
                slots[0] = NB * bs;
                check(ntok == 0 || orc_cache_append(&cd, kn, vn, kc, vc, slots, 1, ks, vs) == -1,
                      "append refuses a slot outside the pool", c);
                void *q = malloc((size_t)B * Hq * D * qb);
                fill(q, (size_t)B * Hq * D, qt);
                orc_decode_desc dd = {B, Hq, Hkv, D, bs, NB, maxb, qt, kt};
                /* room for every row, and for the three rows of the subset call */
                double *out = malloc(sizeof(double) * (size_t)(B * Hq > 3 ? B * Hq : 3) * D);
                const int nth = 1 + (int)rnd(4);
                check(orc_decode(&dd, q, kc, vc, tables, lens, rep == 3 ? starts : NULL,
                                 1.0 / sqrt((double)D), ks, vs, NULL, 0, out, nth) == 0,
                      "decode", c);
                for (size_t i = 0; i < (size_t)B * Hq * D; ++i)
                    check(isfinite(out[i]), "finite output", c);
                for (int h = 0; h < Hq; ++h)
                    for (int d = 0; d < D; ++d)
                        check(out[(size_t)h * D + d] == 0.0, "zero-length row is zero", c);
                /* a row subset, the last rows first */
                int32_t rows[3] = {B * Hq - 1, 0, (B * Hq) / 2};
                check(orc_decode(&dd, q, kc, vc, tables, lens, NULL, 0.125, ks, vs, rows, 3, out,
                                 2) == 0,
                      "decode rows", c);
                /* one-token windows: out = v_scale * V of the window's token */
                int32_t st1[8];
                for (int b = 0; b < B; ++b)
                    st1[b] = lens[b] > 0 ? lens[b] - 1 : 0;
                check(orc_decode(&dd, q, kc, vc, tables, lens, st1, 0.125, ks, vs, NULL, 0, out,
                                 nth) == 0,
                      "decode one-token windows", c);
                for (int b = 1; b < B; ++b) {
                    if (lens[b] == 0)
                        continue;
                    const int p = lens[b] - 1, blk = tables[b * maxb + p / bs];
                    for (int h = 0; h < Hq; ++h) {
                        const int g = h / G;
                        for (int d = 0; d < D; d += 17) {
                            const double want =
                                orc_load(kt, vc, v_index(&(orc_cache_desc){NB, bs, Hkv, D, kt, qt},
                                                         blk, g, p % bs, d)) *
                                vs;
                            check(fabs(out[((size_t)b * Hq + h) * D + d] - want) <=
                                      1e-12 * (1.0 + fabs(want)),
                                  "one-token window value", c);
                        }
                    }
                }
                /* refused: a table entry outside the pool, a bad shape */
                if (B > 1 && lens[B - 1] > 0) {
                    const int32_t keep = tables[(B - 1) * maxb];
                    tables[(B - 1) * maxb] = NB;
                    check(orc_decode(&dd, q, kc, vc, tables, lens, NULL, 0.125, ks, vs, NULL, 0,
                                     out, nth) == -1,
                          "decode refuses an entry outside the pool", c);
                    tables[(B - 1) * maxb] = keep;
                }
                orc_decode_desc bad = dd;
                bad.num_kv_heads = Hq + 1; /* does not divide num_q_heads */
                check(orc_decode(&bad, q, kc, vc, tables, lens, NULL, 0.125, ks, vs, NULL, 0, out,
                                 1) == -3,
                      "decode refuses a bad group", c);
                free(tables); free(perm); free(kc); free(vc); free(kn); free(vn); free(slots);
                free(q); free(out);
            }
    /* the codec over all codes and some floats */
    for (int i = 0; i < 256; ++i)
        (void)orc_e4m3_to_double((uint8_t)i);
    for (int i = -2000; i <= 2000; ++i)
        (void)orc_e4m3_from_float((float)i * 0.37f);
    (void)orc_e4m3_from_float(NAN);
    (void)orc_e4m3_from_float(INFINITY);
    printf("oracle ops: %d cases, %d failed checks\n", c, g_fail);
    return g_fail ? 1 : 0;
}
