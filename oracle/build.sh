#!/bin/sh
# Builds the CPU oracle (test infrastructure) as a shared library beside this script.
set -e
here="$(cd "$(dirname "$0")" && pwd)"
gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off -Wall -Wextra \
    "$here/oracle.c" -o "$here/liboracle.so.tmp" -lm
mv "$here/liboracle.so.tmp" "$here/liboracle.so"
